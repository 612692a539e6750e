"""Build libattn.so (the C-ABI library) for gfx950 with hipcc, in-tree."""

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.hip", "attn_fwd_kernel.hip", "attn_bwd_kernel.hip", "attn_fp8_kernel.hip"]
# the issue-rate microbenchmarks (bench.py --micro) and the exp2_poly accuracy
# kernel: a separate library, not part of the attention ABI
MICRO_LIB = os.path.join(PKG, "libattn_micro.so")
MICRO_SOURCES = ["attn_micro.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument", "-Wl,--no-undefined",
    # packed fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _link(lib, sources, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


def build(verbose=False):
    """Compile every HIP source: the attention library
    (exact_io_aware_27_amd/libattn.so) and the microbenchmark library
    (exact_io_aware_27_amd/libattn_micro.so)."""
    _link(MICRO_LIB, MICRO_SOURCES, verbose)
    return _link(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
