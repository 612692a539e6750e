"""Build libattn.so (the C-ABI library) for gfx950 with hipcc, in-tree."""

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.hip", "attn_fwd_kernel.hip", "attn_bwd_kernel.hip", "attn_fp8_kernel.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument", "-Wl,--no-undefined",
    # packed fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False):
    """Compile every HIP source of the library into exact_io_aware_27_amd/libattn.so."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
