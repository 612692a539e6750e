"""Build libattn.so (the C-ABI library) for gfx950 with hipcc, in-tree."""

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.hip", "attn_fwd_kernel.hip", "attn_decode_kernel.hip", "attn_bwd_kernel.hip", "attn_fp8_kernel.hip"]
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


def _link(lib, sources, verbose, defines=()):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-o", tmp] + srcs
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


def build_variant(out, defines, verbose=False):
    """The attention library with build options (-D NAME=VALUE, e.g.
    ATTN_EXP2_POLY_EVERY=4), written to `out`: for A/B measurements
    (bench.py --lib out)."""
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    return _link(os.path.abspath(out), SOURCES, verbose, defines)


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="build option for a variant library (needs --out)")
    ap.add_argument("--out", default=None, help="path of a variant library")
    a = ap.parse_args()
    if a.out:
        print(build_variant(a.out, a.define, verbose=True))
    else:
        print(build(verbose=True))
