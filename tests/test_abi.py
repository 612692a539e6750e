"""The C ABI without a GPU: the library loads, exports what include/attn.h
declares, and rejects every bad argument before any HIP runtime call."""

import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    from exact_io_aware_27_amd import attn
    if not os.path.exists(attn.LIB_PATH):
        from exact_io_aware_27_amd import build
        build.build()
    return attn.load()


def _declared():
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"ATTN_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_abi():
    assert set(_declared()) == {"attn_fwd", "attn_fwd_splitkv", "attn_fwd_splitkv_workspace_bytes",
                                "attn_fwd_splitkv_noalloc", "attn_noalloc_scratch_bytes",
                                "attn_bwd", "attn_bwd_workspace_bytes", "attn_fp8_padded_rows",
                                "attn_fp8_quantize", "attn_fp8_quantize_q", "attn_fwd_fp8", "attn_status_string",
                                "attn_last_hip_error"}


def test_library_exports_every_declared_symbol(lib):
    from exact_io_aware_27_amd import attn
    out = subprocess.check_output(["nm", "-D", "--defined-only", attn.LIB_PATH], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    names = ["ATTN_OK", "ATTN_NULL_PTR", "ATTN_BAD_SHAPE", "ATTN_UNSUPPORTED_D",
             "ATTN_BAD_SCALE", "ATTN_MISALIGNED", "ATTN_ALIAS", "ATTN_HIP", "ATTN_BAD_WORKSPACE",
             "ATTN_BAD_ARGUMENT", "ATTN_SCRATCH_TOO_SMALL"]
    for code, name in enumerate(names):
        assert lib.attn_status_string(code).decode() == name
    assert lib.attn_status_string(99).decode() == "ATTN_UNKNOWN_STATUS"
    assert lib.attn_last_hip_error() == 0


# Fake, never-dereferenced device addresses: validation fails before any use.
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def _call(lib, q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, N=100, d=128, causal=1, scale=0.1):
    return lib.attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), 2), (dict(H=-5), 2), (dict(N=-1), 2),
    (dict(B=1 << 40, H=1 << 30), 2),              # B*H*N overflows int64
    (dict(N=1 << 24, d=128), 2),                  # N*d = 2^31
    (dict(d=96), 3), (dict(d=256), 3), (dict(d=0), 3),
    (dict(scale=float("nan")), 4), (dict(scale=float("inf")), 4), (dict(scale=-math.inf), 4),
    (dict(B=0, q=None, k=None, v=None, o=None), 0), (dict(N=0), 0), (dict(H=0), 0),
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(q=Q + 8), 5), (dict(o=O + 2), 5), (dict(lse=L + 2), 5),
    (dict(o=Q + 64), 6), (dict(o=K), 6), (dict(lse=V + 16), 6), (dict(lse=O + 1024), 6),
    (dict(d=64, scale=float("nan")), 4), (dict(d=7, B=-1), 2),
])
def test_argument_errors_before_any_hip_call(lib, kw, status):
    assert _call(lib, **kw) == status


def test_lse_null_is_allowed_past_validation_order(lib):
    # With lse NULL the only remaining problem is the alias of o and q.
    assert _call(lib, lse=None, o=Q) == 6


def test_q_k_v_may_alias_each_other(lib):
    # Shared inputs are legal; the only error left is the misaligned output.
    assert _call(lib, k=Q, v=Q, o=O + 4) == 5


W = 0x60000000  # fake workspace address


def _split(lib, q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=7, Nk=1000, d=128, causal=1, scale=0.1,
           S=4, ws=W, wsb=None):
    if wsb is None:
        wsb = lib.attn_fwd_splitkv_workspace_bytes(B, H, Nq, d, S)
    return lib.attn_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, S, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Nq=-1), 2), (dict(Nk=-1), 2), (dict(S=0), 2), (dict(S=-3), 2),
    (dict(Nk=0), 2),                                # queries with no key
    (dict(Nq=1001, Nk=1000), 2),                    # causal: a query would see no key
    (dict(Nk=1 << 24), 2),                          # Nk * d = 2^31
    (dict(d=96), 3), (dict(scale=float("nan")), 4),
    (dict(Nq=0, q=None, o=None, ws=None), 0), (dict(B=0, ws=None), 0),
    (dict(q=None), 1), (dict(k=Q + 8), 5), (dict(o=K + 64), 6), (dict(lse=Q), 6),
    (dict(ws=None), 8), (dict(ws=W + 8), 8), (dict(wsb=100), 8),
    (dict(ws=Q), 8), (dict(ws=L - 64), 8), (dict(ws=O), 8),
])
def test_splitkv_argument_errors_before_any_hip_call(lib, kw, status):
    assert _split(lib, **kw) == status


def test_splitkv_causal_needs_no_more_queries_than_keys_only_under_the_mask(lib):
    # non-causal Nq > Nk passes the shape checks and stops at the misaligned output
    assert _split(lib, Nq=1001, Nk=1000, causal=0, o=O + 4) == 5


def _noalloc(lib, q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=7, Nk=1000, d=128, causal=1, scale=0.1, S=4):
    return lib.attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, S, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Nq=-1), 2), (dict(S=0), 2), (dict(Nk=0), 2), (dict(Nq=1001, Nk=1000), 2),
    (dict(d=96), 3), (dict(scale=float("inf")), 4),
    (dict(Nq=0, q=None, o=None), 0), (dict(H=0), 0),
    (dict(v=None), 1), (dict(o=O + 8), 5), (dict(o=V + 64), 6), (dict(lse=O), 6),
    # the partials of 64 x 32 heads x 128 queries in 8 ranges (1.08 GB) exceed the scratch
    (dict(B=64, H=32, Nq=128, S=8, q=1 << 32, k=2 << 32, v=3 << 32, o=4 << 32, lse=5 << 32), 10),
    # a bad shape is reported before the scratch size
    (dict(B=64, H=32, Nq=128, S=8, d=96), 3),
])
def test_noalloc_argument_errors_before_any_hip_call(lib, kw, status):
    assert _noalloc(lib, **kw) == status


def test_noalloc_scratch_bytes(lib):
    assert lib.attn_noalloc_scratch_bytes() == 32 << 20
    # the largest split call the scratch serves is the one whose workspace fits
    ws = lib.attn_fwd_splitkv_workspace_bytes(2, 3, 7, 128, 4)
    assert 0 < ws <= lib.attn_noalloc_scratch_bytes()


def test_splitkv_workspace_bytes(lib):
    f = lib.attn_fwd_splitkv_workspace_bytes
    assert f(2, 3, 7, 128, 4) == 4 * 2 * 3 * 7 * 129 * 4
    assert f(1, 1, 1, 64, 16) == 16 * 65 * 4
    assert f(2, 3, 7, 128, 1) == 0
    for bad in [(-1, 3, 7, 128, 4), (2, 3, -7, 128, 4), (2, 3, 7, 96, 4), (2, 3, 7, 128, 0),
                (1 << 40, 1 << 20, 1 << 10, 128, 64)]:
        assert f(*bad) == -1


# fake gradient addresses for attn_bwd
G, DQ, DK, DV = 0x70000000, 0x80000000, 0x90000000, 0xA0000000


def _bwd(lib, q=Q, k=K, v=V, o=O, lse=L, g=G, dq=DQ, dk=DK, dv=DV, B=2, H=3, N=100, d=128, causal=1,
         scale=0.1, ws=W, wsb=None):
    if wsb is None:
        wsb = lib.attn_bwd_workspace_bytes(B, H, N, d)
    return lib.attn_bwd(q, k, v, o, lse, g, dq, dk, dv, B, H, N, d, causal, scale, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), 2), (dict(N=-1), 2), (dict(B=1 << 40, H=1 << 30), 2), (dict(N=1 << 24), 2),
    (dict(d=96), 3), (dict(scale=float("nan")), 4), (dict(scale=float("inf")), 4),
    (dict(B=0, q=None, dq=None, ws=None), 0), (dict(N=0, ws=None), 0),
    (dict(q=None), 1), (dict(o=None), 1), (dict(lse=None), 1), (dict(g=None), 1),
    (dict(dq=None), 1), (dict(dk=None), 1), (dict(dv=None), 1),
    (dict(g=G + 8), 5), (dict(dk=DK + 2), 5), (dict(lse=L + 2), 5), (dict(o=O + 4), 5),
    (dict(dq=Q), 6), (dict(dk=O + 64), 6), (dict(dv=G), 6), (dict(dq=L - 64), 6),
    (dict(dk=DQ + 1024), 6), (dict(dv=DK), 6),
    (dict(ws=None), 8), (dict(ws=W + 8), 8), (dict(wsb=100), 8), (dict(ws=DV), 8),
    (dict(ws=L), 8), (dict(ws=G + 256), 8),
])
def test_bwd_argument_errors_before_any_hip_call(lib, kw, status):
    assert _bwd(lib, **kw) == status


def test_bwd_inputs_may_alias_each_other(lib):
    # shared inputs are legal; the only error left is the misaligned dv
    assert _bwd(lib, k=Q, v=Q, o=Q, g=Q, dv=DV + 4) == 5


def test_bwd_workspace_bytes(lib):
    f = lib.attn_bwd_workspace_bytes
    assert f(2, 3, 100, 128) == 2 * 3 * 100 * 8
    assert f(1, 1, 0, 64) == 0
    for bad in [(-1, 3, 7, 128), (2, 3, -7, 128), (2, 3, 7, 96), (1 << 40, 1 << 20, 1 << 10, 128)]:
        assert f(*bad) == -1


def _quant(lib, x=Q, B=2, H=3, N=100, d=128, tr=0, signs=None, out=O, ex=L):
    return lib.attn_fp8_quantize(x, B, H, N, d, tr, signs, out, ex, None)


def _quant_q(lib, x=Q, B=2, H=3, N=100, d=128, signs=None, scale=0.1, out=O, ex=L):
    return lib.attn_fp8_quantize_q(x, B, H, N, d, signs, scale, out, ex, None)


def _fp8(lib, q=Q, k=K, v=V, qe=W, ke=W + 4096, ve=W + 8192, o=O, lse=L, B=2, H=3, N=100, d=128, causal=1):
    return lib.attn_fwd_fp8(q, k, v, qe, ke, ve, o, lse, B, H, N, d, causal, None)


def test_fp8_argument_errors_before_any_hip_call(lib):
    import ctypes
    bits = ctypes.cast((ctypes.c_uint32 * 4)(1, 2, 3, 4), ctypes.c_void_p)
    assert lib.attn_fp8_padded_rows(100) == 128 and lib.attn_fp8_padded_rows(64) == 64
    assert lib.attn_fp8_padded_rows(0) == 0 and lib.attn_fp8_padded_rows(-1) == -1
    assert _quant(lib, B=-1) == 2 and _quant(lib, N=1 << 24) == 2
    assert _quant(lib, d=64) == 3
    assert _quant(lib, tr=1, signs=bits) == 9
    assert _quant(lib, N=0, x=None) == 0
    assert _quant(lib, x=None) == 1 and _quant(lib, ex=None) == 1
    assert _quant(lib, x=Q + 8) == 5 and _quant(lib, out=O + 4) == 5
    assert _quant(lib, out=Q + 64) == 6 and _quant(lib, ex=Q) == 6
    assert _quant_q(lib, B=-1) == 2 and _quant_q(lib, d=64) == 3
    assert _quant_q(lib, scale=float("nan")) == 4 and _quant_q(lib, scale=float("inf"), signs=bits) == 4
    assert _quant_q(lib, N=0, x=None) == 0 and _quant_q(lib, x=None) == 1
    assert _quant_q(lib, out=O + 4) == 5 and _quant_q(lib, ex=Q) == 6
    assert _fp8(lib, N=-1) == 2 and _fp8(lib, d=64) == 3
    assert _fp8(lib, B=0, q=None) == 0
    assert _fp8(lib, q=None) == 1 and _fp8(lib, ve=None) == 1 and _fp8(lib, o=None) == 1
    assert _fp8(lib, k=K + 8) == 5 and _fp8(lib, lse=L + 1) == 5
    assert _fp8(lib, o=Q) == 6 and _fp8(lib, lse=W) == 6 and _fp8(lib, lse=O) == 6


def test_binding_rejects_mismatched_tensors():
    import torch
    from exact_io_aware_27_amd import attn
    x = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.attn_fwd_status(x, x, x, x, None, 1, 2, 8, 128, False, 0.1)
    with pytest.raises(ValueError):
        attn.attn_fwd_status(x.float(), x, x, x, None, 1, 2, 8, 64, False, 0.1)


def test_binding_fails_loudly_without_library(monkeypatch):
    from exact_io_aware_27_amd import attn
    monkeypatch.setattr(attn, "_lib", None)
    monkeypatch.setattr(attn, "LIB_PATH", "/nonexistent/libattn.so")
    with pytest.raises(FileNotFoundError):
        attn.load()


def test_product_and_oracle_share_no_code():
    """Neither side imports, includes or links the other."""
    pkg = os.path.join(ROOT, "exact_io_aware_27_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "attn_oracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert not re.search(r"^\s*(import|from)\s+exact_io_aware_27_amd", text, re.M), f
            includes = re.findall(r"^\s*#\s*include\s*[<\"]([^>\"]+)", text, re.M)
            assert not any("attn.h" in i or "csrc" in i or "attn_launch" in i for i in includes), f
