"""The CPU test tier under AddressSanitizer and UndefinedBehaviorSanitizer.

python tests/sanitize_cpu.py [pytest args]

Builds, into a temporary directory,
  * the C oracles (oracle/attn_oracle.c, oracle/attn_bwd_oracle.c) with clang
    and -fsanitize=address,undefined, and
  * libattn.so with the same sanitizers on its host code only (the argument
    validation and launch code of attn_api.hip and the host side of every
    kernel file; device code is built as usual),
then runs `pytest tests -m "not gpu"` (or the given arguments) in a child
Python with clang's ASan runtime preloaded and ATTN_LIB_PATH /
ATTN_ORACLE_LIB_DIR pointing at the sanitized builds.  UBSan findings abort
(-fno-sanitize-recover); leak checking is off (the interpreter itself is not
instrumented).  The child's exit status is this script's.  Needs no GPU:
every ABI test stops in validation before any HIP call.
"""

import glob
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
       "-fno-omit-frame-pointer"]


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise SystemExit("clang's shared ASan runtime (libclang_rt.asan-x86_64.so) not found")
    return hits[-1]


def build(out):
    from exact_io_aware_27_amd import build as hip_build

    for name in ("attn_oracle", "attn_bwd_oracle"):
        subprocess.check_call(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra"] + SAN +
                              ["-o", os.path.join(out, "lib%s.so" % name), os.path.join(ROOT, "oracle", name + ".c"),
                               "-lm"])
    flags = [f for f in hip_build.FLAGS if f != "-O3"] + ["-O1", "-g"]
    for f in SAN:  # host code only: each sanitizer flag behind -Xarch_host
        flags += ["-Xarch_host", f]
    lib = os.path.join(out, "libattn.so")
    subprocess.check_call([hip_build.HIPCC] + flags + ["-o", lib] +
                          [os.path.join(hip_build.CSRC, s) for s in hip_build.SOURCES])
    return lib


def main(argv):
    with tempfile.TemporaryDirectory(prefix="attn_san_") as out:
        lib = build(out)
        env = dict(os.environ, LD_PRELOAD=asan_runtime(), ATTN_LIB_PATH=lib, ATTN_ORACLE_LIB_DIR=out,
                   ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        args = argv or [os.path.join(ROOT, "tests"), "-m", "not gpu", "-q", "-p", "no:cacheprovider"]
        # the preload instruments this interpreter; child processes the tests
        # start (gcc, hipcc, nm) run without it
        code = ("import os, sys; os.environ.pop('LD_PRELOAD', None); import pytest; "
                "sys.exit(pytest.main(%r))" % (args,))
        return subprocess.call([sys.executable, "-c", code], env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
