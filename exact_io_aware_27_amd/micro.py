"""ctypes binding of libattn_micro.so: the gfx950 issue-rate microbenchmarks
(csrc/attn_micro.hip) and the exp2_poly accuracy kernel.  Measurement tools,
not part of the attention ABI.  Raises if the library is not built."""

import ctypes
import os

import torch  # noqa: F401  (loaded first: one HIP runtime per process)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_micro.so")
OPS = {"fma": 0, "exp": 1, "poly": 2, "mul": 3}
# VALU instructions per loop element of each rate op: exp2_poly applied to -x
# is the negation plus its 8 instructions; v_exp_f32 takes the negation as an
# input modifier.
INSTS_PER_OP = {"fma": 1, "exp": 1, "poly": 9, "mul": 1}
MIXES = [(0, 0, False), (2, 1, False), (3, 1, False), (4, 1, False), (5, 1, False), (6, 1, False),
         (4, 2, False), (8, 0, False), (3, 1, True), (4, 1, True)]

_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError("libattn_micro.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    d4 = ctypes.POINTER(ctypes.c_double)
    lib.attn_micro_rate.restype = ctypes.c_int
    lib.attn_micro_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, d4]
    lib.attn_micro_mix.restype = ctypes.c_int
    lib.attn_micro_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, d4]
    lib.attn_micro_mix_shape.restype = ctypes.c_int
    lib.attn_micro_mix_shape.argtypes = [ctypes.c_int] * 6 + [d4]
    lib.attn_micro_lds_rate.restype = ctypes.c_int
    lib.attn_micro_lds_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, d4]
    lib.attn_micro_mix_lds.restype = ctypes.c_int
    lib.attn_micro_mix_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, d4]
    lib.attn_micro_hbm_read.restype = ctypes.c_int
    lib.attn_micro_hbm_read.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, d4]
    lib.attn_micro_exp2.restype = ctypes.c_int
    lib.attn_micro_exp2.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    _lib = lib
    return lib


def rate(op, waves_per_simd, dependent=False, iters=20000):
    """Cycles per instruction of one VALU op kind: per SIMD over all its waves
    (independent chains) or per dependent instruction (one chain); and the
    measured shader clock (GHz)."""
    out = (ctypes.c_double * 4)()
    st = load().attn_micro_rate(OPS[op], 1 if dependent else 0, waves_per_simd, iters, out)
    if st:
        raise RuntimeError("attn_micro_rate status %d" % st)
    return {"op": op, "waves_per_simd": waves_per_simd, "dependent": dependent,
            "cycles_per_element": out[0], "cycles_per_inst": out[0] / INSTS_PER_OP[op],
            "clock_ghz": out[1], "ms": out[2]}


SHAPES = {0: "independent", 1: "one MFMA accumulator chain", 2: "each exp on the FMA before it"}
SHAPED_MIXES = [(0, 0, 1), (4, 1, 1), (4, 1, 2)]


def mix(k_fma, n_exp, poly, waves_per_simd, iters=20000, shape=0):
    """Cycles per 32x32x16 bf16 MFMA per SIMD with k_fma FMAs and n_exp
    exponentials after each MFMA (32 = the matrix core's own rate); shape
    as SHAPES."""
    out = (ctypes.c_double * 4)()
    st = load().attn_micro_mix_shape(k_fma, n_exp, 1 if poly else 0, shape, waves_per_simd, iters, out)
    if st:
        raise RuntimeError("attn_micro_mix status %d" % st)
    return {"k_fma": k_fma, "n_exp": n_exp, "exp": "exp2_poly" if poly else "v_exp_f32", "shape": SHAPES[shape],
            "waves_per_simd": waves_per_simd, "cycles_per_mfma": out[0], "clock_ghz": out[1],
            "ms": out[2], "tflops": out[3]}


LDS_READS = {0: "ds_read_b128", 1: "ds_read_b64_tr_b16"}
LDS_OPERANDS = {0: "ds_read_b128", 1: "2 x ds_read_b64_tr_b16",
                2: "ds_read_b128 for 8 MFMAs, 2 x ds_read_b64_tr_b16 for 8 (the attention step)"}


def lds_rate(kind, waves_per_simd, iters=20000):
    """LDS read throughput of one read kind (0 ds_read_b128, 1
    ds_read_b64_tr_b16) on consecutive addresses: bytes per shader cycle per
    CU over all its waves, and the shader clock (GHz)."""
    out = (ctypes.c_double * 4)()
    st = load().attn_micro_lds_rate(kind, waves_per_simd, iters, out)
    if st:
        raise RuntimeError("attn_micro_lds_rate status %d" % st)
    return {"read": LDS_READS[kind], "waves_per_simd": waves_per_simd, "bytes_per_cycle_per_cu": out[0],
            "clock_ghz": out[1], "ms": out[2]}


def mix_lds(kind, waves_per_simd, iters=20000):
    """Cycles per 32x32x16 bf16 MFMA per SIMD when each MFMA's A operand (1 KB
    a wave) is read from LDS in the attention step's issue order (kind as
    LDS_OPERANDS), with no VALU work; one or two waves per SIMD."""
    out = (ctypes.c_double * 4)()
    st = load().attn_micro_mix_lds(kind, waves_per_simd, iters, out)
    if st:
        raise RuntimeError("attn_micro_mix_lds status %d" % st)
    return {"operand": LDS_OPERANDS[kind], "waves_per_simd": waves_per_simd, "cycles_per_mfma": out[0],
            "clock_ghz": out[1], "ms": out[2], "tflops": out[3]}


def hbm_read(mib, wgs, blocked=False, reps=10):
    """GB/s of a plain 16-byte-per-thread read stream over `mib` MiB on
    `wgs` workgroups of 256 threads, grid-interleaved or (blocked) one
    contiguous slice per workgroup (the last of `reps` launches)."""
    out = (ctypes.c_double * 4)()
    st = load().attn_micro_hbm_read(mib, wgs, reps, 1 if blocked else 0, out)
    if st:
        raise RuntimeError("attn_micro_hbm_read status %d" % st)
    return {"mib": mib, "workgroups": wgs, "blocked": blocked, "GBps": out[0], "ms": out[1]}


def exp2(x, stream=None):
    """(exp2_poly(x), v_exp_f32(x)) elementwise for a contiguous fp32 CUDA tensor."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 CUDA tensor")
    poly, hw = torch.empty_like(x), torch.empty_like(x)
    s = stream.cuda_stream if stream is not None else torch.cuda.current_stream(x.device).cuda_stream
    st = load().attn_micro_exp2(x.data_ptr(), poly.data_ptr(), hw.data_ptr(), x.numel(), s)
    if st:
        raise RuntimeError("attn_micro_exp2 status %d" % st)
    return poly, hw
