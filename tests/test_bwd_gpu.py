"""Backward pass (attn_bwd) against the fp64 backward oracle, on a GPU.

The kernels recompute P from the forward pass's LSE and take D from its O, so
every case runs attn_fwd first and hands its (O, LSE) to attn_bwd, as a
training step does.  Expected values come from oracle.attention_bwd (the
plain derivative of the forward definition, fp64); inputs are seeded and
synthetic.  The bar is stated in tests/parity.py (compare_grad).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_27_amd import inputs
import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def case(B, H, N, d, seed):
    q, k, v = inputs.make_qkv(B, H, N, d, seed=seed)
    g = inputs.make_grad_out(B, H, N, d, seed=seed + 104729)
    return q, k, v, g


def run(q, k, v, g, causal, scale, workspace=None):
    from exact_io_aware_27_amd import attn
    qd, kd, vd, gd = (x.to(DEV) for x in (q, k, v, g))
    o, lse = attn.attention(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = attn.attention_bwd(qd, kd, vd, o, lse, gd, causal=causal, scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(q, k, v, g, causal, scale, what):
    say("case:", what, tuple(q.shape), "causal" if causal else "non-causal", "scale %.4g" % scale)
    dq, dk, dv = run(q, k, v, g, causal, scale)
    rq, rk, rv, _ = oracle.attention_bwd(q, k, v, g, causal, scale)
    for name, x, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        rep = parity.compare_grad(x, ref)
        say("  ", name, rep)
        parity.assert_grad_parity(rep, "%s %s" % (what, name))
    return dq, dk, dv


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 2, 256, 64, False), (1, 2, 256, 128, True), (2, 1, 200, 128, True), (1, 2, 200, 64, False),
    (1, 1, 1, 64, True), (1, 1, 1, 128, False), (1, 3, 129, 64, True), (1, 1, 700, 128, False),
    (1, 2, 1000, 64, True), (1, 1, 513, 128, True), (2, 2, 64, 128, False), (1, 1, 33, 64, True)])
def test_matches_oracle(B, H, N, d, causal):
    q, k, v, g = case(B, H, N, d, seed=3000 + N + d + causal)
    check(q, k, v, g, causal, 1.0 / math.sqrt(d), "B=%d H=%d N=%d d=%d" % (B, H, N, d))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 129, 777])
def test_small_causal_grid_single_blocks_longest_first(d, N):
    """8 | B H and too few heavy+light pairs to fill the chip twice: both
    kernels run single blocks, longest first within each XCD (the dQ kernel
    from the last query block, the dK/dV kernel from the first key block)."""
    q, k, v, g = case(2, 4, N, d, seed=7000 + N + d)
    check(q, k, v, g, True, 1.0 / math.sqrt(d), "B=2 H=4 N=%d d=%d causal" % (N, d))


def test_gpt2_small_shape_every_head():
    # 8 x 12 heads of 1024 queries, d = 64, causal: the GPT-2 (seq 1K) shape
    w = [x for x in inputs.WORKLOADS if x.name == "gpt2_small"][0]
    q, k, v, g = case(w.B, w.H, w.N, w.d, seed=w.seed)
    check(q, k, v, g, w.causal, w.scale, "gpt2_small")


def test_scale_argument_is_used():
    q, k, v, g = case(1, 2, 300, 128, seed=3101)
    check(q, k, v, g, False, 0.37, "scale 0.37")
    check(q, k, v, g, True, 0.02, "scale 0.02")
    check(q, k, v, g, True, -0.2, "scale -0.2")


def test_long_causal_one_head_and_invariants_of_all():
    """The full B=2 H=32 N=8192 d=128 causal shape: one head against the
    oracle element by element, and for every head the identities that hold at
    any size: each row of dS sums to zero, so sum_j dK_j = 0, and each row of P
    sums to one, so sum_j dV_j = sum_i dO_i."""
    w = [x for x in inputs.WORKLOADS if x.name == "long_causal"][0]
    q, k, v = inputs.workload_qkv(w)
    g = inputs.make_grad_out(w.B, w.H, w.N, w.d, seed=w.seed + 104729)
    say("case: long_causal", (w.B, w.H, w.N, w.d))
    dq, dk, dv = run(q, k, v, g, w.causal, w.scale)
    b, h = 1, 17
    sl = (slice(b, b + 1), slice(h, h + 1))
    rq, rk, rv, _ = oracle.attention_bwd(q[sl], k[sl], v[sl], g[sl], w.causal, w.scale)
    for name, x, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        rep = parity.compare_grad(x[sl], ref)
        say("  head (%d, %d)" % (b, h), name, rep)
        parity.assert_grad_parity(rep, "long_causal %s" % name)
    dk64, dv64 = dk.double(), dv.double()
    # each sum has N terms of bf16-rounded outputs: compare with the sum of |terms|
    ksum = dk64.sum(dim=2).abs() / dk64.abs().sum(dim=2).clamp_min(1e-30)
    vsum = (dv64.sum(dim=2) - g.to(DEV).double().sum(dim=2)).abs() / dv64.abs().sum(dim=2).clamp_min(1e-30)
    say("   invariants: max rel |sum dK| %.3g, max rel |sum dV - sum dO| %.3g" % (ksum.max(), vsum.max()))
    assert float(ksum.max()) < 1e-2 and float(vsum.max()) < 1e-2


def test_deterministic_and_workspace_reusable():
    q, k, v, g = case(1, 4, 777, 128, seed=3102)
    ws = torch.empty(8 * 4 * 777 + 256, dtype=torch.uint8, device=DEV)
    a = run(q, k, v, g, True, 0.1, workspace=ws)
    b = run(q, k, v, g, True, 0.1, workspace=ws)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("d", [64, 128])
def test_every_output_element_is_written(d):
    from exact_io_aware_27_amd import attn
    B, H, N = 1, 3, 333
    q, k, v, g = (x.to(DEV) for x in case(B, H, N, d, seed=3103 + d))
    o, lse = attn.attention(q, k, v, causal=True)
    outs = [torch.full_like(q, float("nan")) for _ in range(3)]
    nb = attn.bwd_workspace_bytes(B, H, N, d)
    ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=DEV)
    attn.attn_bwd(q, k, v, o, lse, g, *outs, B, H, N, d, True, d ** -0.5, ws, nb, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for x in outs:
        assert bool(torch.isfinite(x.float()).all())


@pytest.mark.parametrize("N,d,causal", [(100, 64, True), (200, 128, False), (65, 128, True)])
def test_memory_past_the_sequence_is_never_read(N, d, causal):
    """Every operand of the last head sits at the start of a NaN-filled
    allocation (the workspace too), so any row read past N would turn the
    gradients into NaN through 0 * NaN."""
    from exact_io_aware_27_amd import attn
    B, H = 1, 2
    q, k, v, g = case(B, H, N, d, seed=3200 + N + d)
    scale = 1.0 / math.sqrt(d)
    say("case: NaN past the end", (B, H, N, d), "causal" if causal else "non-causal")
    n = B * H * N * d
    pad = 64 * 1024 * d

    def padded(x):
        big = torch.full((n + pad,), float("nan"), dtype=torch.bfloat16, device=DEV)
        big[:n].copy_(x.reshape(-1).to(DEV))
        return big[:n].view(B, H, N, d)

    qd, kd, vd, gd = padded(q), padded(k), padded(v), padded(g)
    o = padded(torch.zeros(B, H, N, d, dtype=torch.bfloat16))
    lse_big = torch.full((B * H * N + 65536,), float("nan"), dtype=torch.float32, device=DEV)
    lse = lse_big[:B * H * N].view(B, H, N)
    attn.attn_fwd(qd, kd, vd, o, lse, B, H, N, d, causal, scale, torch.cuda.current_stream())
    nb = attn.bwd_workspace_bytes(B, H, N, d)
    ws = torch.full((nb // 4 + 65536,), float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    attn.attn_bwd(qd, kd, vd, o, lse, gd, dq, dk, dv, B, H, N, d, causal, scale, ws, nb,
                  torch.cuda.current_stream())
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_bwd(q, k, v, g, causal, scale)
    for name, x, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        rep = parity.compare_grad(x, ref)
        say("  ", name, rep)
        parity.assert_grad_parity(rep, "NaN past the end %s" % name)


def test_single_key_closed_form():
    """N = 1: P = 1 (its bf16 rounding is exactly 1), so dV = dO bit for bit,
    and dS = dP - D = dO.v - dO.O with O = v is zero up to the fp32 order of
    two sums of the same products."""
    q, k, v, g = case(2, 3, 1, 128, seed=3300)
    dq, dk, dv = run(q, k, v, g, True, 0.125)
    assert float(dq.float().abs().max()) < 1e-4 and float(dk.float().abs().max()) < 1e-4
    assert torch.equal(dv.cpu().view(torch.int16), g.view(torch.int16))


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_very_long_sequence_sampled_dq_rows_and_identities(d, causal):
    """N = 65536: sampled dQ rows element by element against the oracle's
    row-by-row entry (O(N d) per row), held to the rounding model of long sums
    (tests/parity.py, compare_grad_model), and for dK and dV the identities
    that hold at any size."""
    B, H, N = 1, 2, 65536
    q, k, v, g = case(B, H, N, d, seed=3400 + d)
    scale = 1.0 / math.sqrt(d)
    say("case: very long", (B, H, N, d), "causal" if causal else "non-causal")
    dq, dk, dv = run(q, k, v, g, causal, scale)
    rows = torch.stack([inputs.row_subset(N, 24, 3400, bh, (0, 1, N - 1)) for bh in range(B * H)])
    rq, _, term2, pk, o, pv2 = oracle.attention_bwd_dq_rows(q, k, v, g, causal, scale, rows.numpy(),
                                                            with_terms=True)
    g_rows = parity.gather_rows(g, rows).double().numpy()
    rep = parity.compare_grad_model(parity.gather_rows(dq, rows), rq, term2, pk, o, g_rows, scale, pv2)
    say("   sampled dQ rows", rep)
    parity.assert_grad_model(rep, "very long dQ rows")
    dk64, dv64 = dk.double(), dv.double()
    ksum = dk64.sum(dim=2).abs() / dk64.abs().sum(dim=2).clamp_min(1e-30)
    vsum = (dv64.sum(dim=2) - g.to(DEV).double().sum(dim=2)).abs() / dv64.abs().sum(dim=2).clamp_min(1e-30)
    say("   invariants: max rel |sum dK| %.3g, max rel |sum dV - sum dO| %.3g" % (ksum.max(), vsum.max()))
    assert float(ksum.max()) < 1e-2 and float(vsum.max()) < 1e-2
