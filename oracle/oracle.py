"""ctypes front end of the fp64 C oracles (``attn_oracle.c``, ``attn_bwd_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Parity of the forward
is pinned in tests/test_oracle.py: closed forms, PyTorch's CPU
``scaled_dot_product_attention`` in float64, and the two-block merge identity
of "FlashAttention evolution" (letsgetai.github.io), section on the core
mechanism, merge equation.  Parity of the gradients is pinned in
tests/test_bwd_oracle.py: PyTorch autograd in float64, central finite
differences and closed forms.
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_BWD_SRC = os.path.join(_HERE, "attn_bwd_oracle.c")
# ATTN_ORACLE_LIB_DIR: a directory holding prebuilt libattn_oracle.so and
# libattn_bwd_oracle.so of the same sources (the sanitizer build of
# tests/sanitize_cpu.py); by default the libraries are built here.
_PREBUILT = os.environ.get("ATTN_ORACLE_LIB_DIR")
_LIB = os.path.join(_PREBUILT or _HERE, "libattn_oracle.so")
_BWD_LIB = os.path.join(_PREBUILT or _HERE, "libattn_bwd_oracle.so")
_lib = None
_bwd_lib = None

ORACLE_STATUS = {0: "OK", 1: "BAD_ARG", 2: "NO_MEMORY", 3: "PSUM"}


def library_path():
    return _LIB


def _compile(src, lib, force):
    if _PREBUILT:
        return lib  # a prebuilt library of the same source is in use
    if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(src):
        return lib
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


def build(force=True):
    """Compile the C oracles with gcc into oracle/libattn_oracle.so and
    oracle/libattn_bwd_oracle.so.

    Plain -O2, no -ffast-math and no -march, so fp64 arithmetic keeps its
    IEEE meaning and the libraries run on any x86-64 host.
    """
    _compile(_BWD_SRC, _BWD_LIB, force)
    return _compile(_SRC, _LIB, force)


def load_library(path):
    """Open a compiled oracle library and declare oracle_attn_qk's signature."""
    lib = ctypes.CDLL(path)
    f = lib.oracle_attn_qk
    f.restype = ctypes.c_int
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    f.argtypes = [p, p, p, i64, i64, i64, i64, ctypes.c_int, ctypes.c_double,
                  p, i64, p, p, p, ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        _compile(_SRC, _LIB, force=False)
        _lib = load_library(_LIB)
    return _lib


def load_bwd_library(path):
    """Open a compiled backward oracle and declare oracle_attn_bwd's signature."""
    lib = ctypes.CDLL(path)
    f = lib.oracle_attn_bwd
    f.restype = ctypes.c_int
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    f.argtypes = [p, p, p, p, i64, i64, i64, i64, ctypes.c_int, ctypes.c_double,
                  p, p, p, p, ctypes.c_int]
    g = lib.oracle_attn_bwd_dq_rows
    g.restype = ctypes.c_int
    g.argtypes = [p, p, p, p, i64, i64, i64, i64, ctypes.c_int, ctypes.c_double, p, i64, p, p, p, p, p, p]
    return lib


def _load_bwd():
    global _bwd_lib
    if _bwd_lib is None:
        _compile(_BWD_SRC, _BWD_LIB, force=False)
        _bwd_lib = load_bwd_library(_BWD_LIB)
    return _bwd_lib


def default_threads():
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _bf16_bits(x):
    """bf16 bit patterns as a contiguous uint16 array (torch bf16 tensor or uint16 array)."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("numpy input must hold bf16 bit patterns as uint16")
        return np.ascontiguousarray(x)
    import torch  # only for the bf16 -> bits view of a CPU tensor

    if x.dtype != torch.bfloat16:
        raise TypeError("torch input must be bfloat16")
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def attention(q, k, v, causal, scale, rows=None, nthreads=None, return_psum_dev=False, lib=None):
    """Exact attention in fp64 for bf16 q [B, H, Nq, d] and k, v [B, H, Nk, d].

    Under the causal mask query i sees key j iff j <= i + (Nk - Nq): the
    queries are the last Nq positions of the key sequence (Nq <= Nk).
    rows: None for every query row, else an int array [B*H, R] (or [B, H, R])
    of query indices per (batch, head).
    Returns (o, lse): o float64 [B, H, R, d], lse float64 [B, H, R]
    (and psum_dev float64 [B, H, R], |sum_j P_ij - 1|, if asked).
    lib: a library from load_library() to use instead of the built one.
    """
    qb, kb, vb = _bf16_bits(q), _bf16_bits(k), _bf16_bits(v)
    if qb.ndim != 4 or kb.shape != vb.shape or kb.ndim != 4 or qb.shape[:2] != kb.shape[:2] \
            or qb.shape[3] != kb.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v one [B, H, Nk, d] shape")
    B, H, Nq, d = qb.shape
    Nk = kb.shape[2]
    BH = B * H
    if rows is None:
        R = Nq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(BH, -1))
        R = rows_arr.shape[1]
    o = np.empty((BH, R, d), dtype=np.float64)
    lse = np.empty((BH, R), dtype=np.float64)
    dev = np.empty((BH, R), dtype=np.float64)
    lib = lib or _load()
    st = lib.oracle_attn_qk(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, BH, Nq, Nk, d,
                            1 if causal else 0, float(scale),
                            None if rows_arr is None else rows_arr.ctypes.data, R,
                            o.ctypes.data, lse.ctypes.data, dev.ctypes.data,
                            int(nthreads or default_threads()))
    if st != 0:
        raise RuntimeError("oracle_attn failed: %s" % ORACLE_STATUS.get(st, st))
    out = (o.reshape(B, H, R, d), lse.reshape(B, H, R))
    if return_psum_dev:
        out = out + (dev.reshape(B, H, R),)
    return out


def attention_bwd(q, k, v, do, causal, scale, nthreads=None, lib=None):
    """Gradients of exact attention in fp64 for bf16 q, do [B, H, Nq, d] and
    k, v [B, H, Nk, d] (causal: Nq <= Nk, query i sees key j iff
    j <= i + Nk - Nq).

    Returns (dq, dk, dv, dsum): float64 [B, H, Nq, d], [B, H, Nk, d] twice,
    and D = rowsum(dO * O) as float64 [B, H, Nq].
    lib: a library from load_bwd_library() to use instead of the built one.
    """
    qb, kb, vb, gb = _bf16_bits(q), _bf16_bits(k), _bf16_bits(v), _bf16_bits(do)
    if qb.ndim != 4 or kb.ndim != 4 or kb.shape != vb.shape or gb.shape != qb.shape \
            or qb.shape[:2] != kb.shape[:2] or qb.shape[3] != kb.shape[3]:
        raise ValueError("q, do must be [B, H, Nq, d] and k, v one [B, H, Nk, d] shape")
    B, H, Nq, d = qb.shape
    Nk = kb.shape[2]
    BH = B * H
    dq = np.empty((BH, Nq, d), dtype=np.float64)
    dk = np.empty((BH, Nk, d), dtype=np.float64)
    dv = np.empty((BH, Nk, d), dtype=np.float64)
    dsum = np.empty((BH, Nq), dtype=np.float64)
    lib = lib or _load_bwd()
    st = lib.oracle_attn_bwd(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, gb.ctypes.data,
                             BH, Nq, Nk, d, 1 if causal else 0, float(scale),
                             dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, dsum.ctypes.data,
                             int(nthreads or default_threads()))
    if st != 0:
        raise RuntimeError("oracle_attn_bwd failed: %s" % ORACLE_STATUS.get(st, st))
    return (dq.reshape(B, H, Nq, d), dk.reshape(B, H, Nk, d), dv.reshape(B, H, Nk, d),
            dsum.reshape(B, H, Nq))


def attention_bwd_dq_rows(q, k, v, do, causal, scale, rows, lib=None, with_terms=False):
    """dQ (and D) of the query rows `rows` (int array [B*H, R] or [B, H, R])
    of every head, fp64, row by row.  Returns (dq [B, H, R, d], dsum [B, H, R])
    and, with_terms, term2, pk, o, pv2 [B, H, R, d]: sum_j (scale dS_ij k_jt)^2,
    sum_j P_ij k_jt, the output row O_i and sum_j P_ij^2 (v_jt - O_it)^2."""
    qb, kb, vb, gb = _bf16_bits(q), _bf16_bits(k), _bf16_bits(v), _bf16_bits(do)
    B, H, Nq, d = qb.shape
    Nk = kb.shape[2]
    BH = B * H
    rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(BH, -1))
    R = rows_arr.shape[1]
    dq = np.empty((BH, R, d), dtype=np.float64)
    dsum = np.empty((BH, R), dtype=np.float64)
    term2 = np.empty((BH, R, d), dtype=np.float64) if with_terms else None
    pk = np.empty((BH, R, d), dtype=np.float64) if with_terms else None
    o = np.empty((BH, R, d), dtype=np.float64) if with_terms else None
    pv2 = np.empty((BH, R, d), dtype=np.float64) if with_terms else None
    lib = lib or _load_bwd()
    st = lib.oracle_attn_bwd_dq_rows(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, gb.ctypes.data, BH, Nq, Nk,
                                     d, 1 if causal else 0, float(scale), rows_arr.ctypes.data, R,
                                     dq.ctypes.data, dsum.ctypes.data,
                                     None if term2 is None else term2.ctypes.data,
                                     None if pk is None else pk.ctypes.data,
                                     None if o is None else o.ctypes.data,
                                     None if pv2 is None else pv2.ctypes.data)
    if st != 0:
        raise RuntimeError("oracle_attn_bwd_dq_rows failed: %s" % ORACLE_STATUS.get(st, st))
    out = (dq.reshape(B, H, R, d), dsum.reshape(B, H, R))
    if with_terms:
        out = out + tuple(x.reshape(B, H, R, d) for x in (term2, pk, o, pv2))
    return out
