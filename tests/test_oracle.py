"""Pins of the fp64 oracle to things other than itself.

Each test is chosen so a plausible slip in the oracle fails at least one:
  dropped or doubled scale        -> SDPA, equal keys (LSE), golden cases
  missing max subtraction         -> golden huge-logit case (fp64 overflow)
  causal direction / off-by-one   -> SDPA causal, causal row 0, equal keys
  transposed operand / wrong V    -> SDPA, one-hot dominant logits
  LSE in the wrong base           -> equal keys, golden, merge identity
  missing final 1/l               -> every closed form
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from exact_io_aware_27_amd import inputs
import golden_cases


def _wide(x):
    return x.to(torch.float64)


def _sdpa64(q, k, v, causal, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        _wide(q), _wide(k), _wide(v), is_causal=causal, scale=scale).numpy()


def _lse_scipy(q, k, causal, scale):
    s = scale * np.einsum("bhid,bhjd->bhij", _wide(q).numpy(), _wide(k).numpy())
    if causal:
        N = s.shape[-1]
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    return scipy.special.logsumexp(s, axis=-1)


@pytest.mark.parametrize("N,d,causal", [
    (256, 64, False), (256, 64, True), (1, 64, False), (1, 128, True), (7, 64, True),
    (63, 128, False), (65, 128, True), (200, 64, False), (200, 128, True)])
def test_matches_torch_sdpa_float64(N, d, causal):
    q, k, v = inputs.make_qkv(1, 2, N, d, seed=100 + N + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, causal, scale)
    np.testing.assert_allclose(o, _sdpa64(q, k, v, causal, scale), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _lse_scipy(q, k, causal, scale), rtol=0, atol=1e-12)


def test_tiny_workload_matches_sdpa_and_p_rows_sum_to_one():
    w = inputs.WORKLOADS[0]
    q, k, v = inputs.workload_qkv(w)
    o, lse, dev = oracle.attention(q, k, v, w.causal, w.scale, return_psum_dev=True)
    np.testing.assert_allclose(o, _sdpa64(q, k, v, w.causal, w.scale), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _lse_scipy(q, k, w.causal, w.scale), rtol=0, atol=1e-12)
    assert dev.max() <= 1e-12


@pytest.mark.parametrize("case", golden_cases.load(), ids=lambda c: c["name"])
def test_golden_worked_cases(case):
    N = case["N"]
    o, lse = oracle.attention(case["q"], case["k"], case["v"], case["causal"], case["scale"])
    np.testing.assert_allclose(o[0, 0], case["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], case["lse"], rtol=1e-15, atol=1e-13)
    assert o.shape == (1, 1, N, case["d"])


@pytest.mark.parametrize("causal", [False, True])
def test_equal_keys_give_mean_of_visible_values(causal):
    N, d = 97, 128
    q, _, v = inputs.make_qkv(1, 1, N, d, seed=7)
    krow = inputs.make_qkv(1, 1, 1, d, seed=8)[1]
    k = krow.expand(1, 1, N, d).contiguous()
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, causal, scale)
    vv = _wide(v)[0, 0].numpy()
    s = scale * (_wide(q)[0, 0].numpy() @ _wide(krow)[0, 0, 0].numpy())
    for i in range(N):
        n = i + 1 if causal else N
        np.testing.assert_allclose(o[0, 0, i], vv[:n].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, i] - (s[i] + math.log(n))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_one_hot_dominant_logits_select_one_value_row(causal):
    N, d = 64, 128
    _, k, v = inputs.make_qkv(1, 1, N, d, seed=11)
    g = torch.Generator().manual_seed(12)
    perm = torch.arange(N) if causal else torch.randperm(N, generator=g)
    q = (k[0, 0, perm] * 16).reshape(1, 1, N, d)  # times a power of two: exact in bf16
    scale = 1.0 / math.sqrt(d)
    o, _ = oracle.attention(q, k, v, causal, scale)
    s = scale * (_wide(q)[0, 0].numpy() @ _wide(k)[0, 0].numpy().T)
    vv = _wide(v)[0, 0].numpy()
    for i in range(N):
        vis = np.arange(i + 1) if causal else np.arange(N)
        j = int(perm[i])
        others = s[i, vis[vis != j]]
        margin = s[i, j] - (others.max() if others.size else -np.inf)
        assert margin >= 40
        bound = (len(vis) - 1) * math.exp(-margin) * 2 * np.abs(vv).max() + 1e-15
        np.testing.assert_allclose(o[0, 0, i], vv[j], rtol=0, atol=bound)


def test_causal_row_zero_is_first_value_row():
    N, d = 129, 64
    q, k, v = inputs.make_qkv(2, 3, N, d, seed=13)
    scale = 0.125
    o, lse = oracle.attention(q, k, v, True, scale)
    assert np.array_equal(o[:, :, 0], _wide(v)[:, :, 0].numpy())
    dots = scale * (_wide(q)[:, :, 0] * _wide(k)[:, :, 0]).sum(-1).numpy()
    np.testing.assert_allclose(lse[:, :, 0], dots, rtol=0, atol=1e-13)


def test_single_key_returns_value():
    q, k, v = inputs.make_qkv(1, 4, 1, 128, seed=14)
    o, lse = oracle.attention(q, k, v, False, 0.3)
    assert np.array_equal(o[:, :, 0], _wide(v)[:, :, 0].numpy())
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * (_wide(q) * _wide(k)).sum(-1)[:, :, 0].numpy(),
                               rtol=0, atol=1e-13)


def test_key_value_permutation_invariance_noncausal():
    N, d = 150, 64
    q, k, v = inputs.make_qkv(1, 2, N, d, seed=15)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(16))
    o1, l1 = oracle.attention(q, k, v, False, 0.125)
    o2, l2 = oracle.attention(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), False, 0.125)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_two_block_merge_identity_on_oracle_halves():
    """Oracle on key halves, merged with the pages' merge equation, equals the full run."""
    N, d = 300, 128
    q, k, v = inputs.make_qkv(1, 2, N, d, seed=17, sigma_qk=3.0)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, False, scale)
    h = 137
    o1, l1 = _partial(q, k[:, :, :h], v[:, :, :h], scale)
    o2, l2 = _partial(q, k[:, :, h:], v[:, :, h:], scale)
    om, lm = oracle.merge_partials(o1, l1, o2, l2)
    np.testing.assert_allclose(om, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, lse, rtol=0, atol=1e-12)


def _partial(q, k, v, scale):
    """Every query row of q against the key subset (k, v), non-causal.

    The oracle takes square problems, so the queries are fed in chunks of
    Nk rows (the last chunk zero-padded) and only the real rows are kept.
    """
    BH, Nq, Nk = q.shape[0] * q.shape[1], q.shape[2], k.shape[2]
    outs_o, outs_l = [], []
    for r0 in range(0, Nq, Nk):
        n = min(Nq, r0 + Nk) - r0
        qq = torch.zeros(q.shape[0], q.shape[1], Nk, q.shape[3], dtype=q.dtype)
        qq[:, :, :n] = q[:, :, r0:r0 + n]
        rows = np.tile(np.arange(n, dtype=np.int64), (BH, 1))
        o, l = oracle.attention(qq, k.contiguous(), v.contiguous(), False, scale, rows=rows)
        outs_o.append(o)
        outs_l.append(l)
    return np.concatenate(outs_o, axis=2), np.concatenate(outs_l, axis=2)


def test_value_scaling_by_two_is_exact():
    q, k, v = inputs.make_qkv(1, 1, 80, 64, seed=18)
    o1, l1 = oracle.attention(q, k, v, True, 0.125)
    o2, l2 = oracle.attention(q, k, (v.float() * 2).to(torch.bfloat16), True, 0.125)
    assert np.array_equal(o2, 2 * o1) and np.array_equal(l1, l2)


def test_row_subset_matches_full_run():
    N, d = 300, 64
    q, k, v = inputs.make_qkv(1, 3, N, d, seed=19)
    rows = torch.stack([inputs.row_subset(N, 40, 19, bh, (0, N - 1)) for bh in range(3)])
    o, lse = oracle.attention(q, k, v, True, 0.125)
    os_, ls = oracle.attention(q, k, v, True, 0.125, rows=rows)
    for bh in range(3):
        assert np.array_equal(os_[0, bh], o[0, bh, rows[bh].numpy()])
        assert np.array_equal(ls[0, bh], lse[0, bh, rows[bh].numpy()])


def test_rejects_bad_rows():
    q, k, v = inputs.make_qkv(1, 1, 8, 64, seed=20)
    with pytest.raises(RuntimeError):
        oracle.attention(q, k, v, False, 0.1, rows=np.array([[8]]))


# ---- fewer queries than keys (queries are the last Nq positions) ----

def _sdpa64_mask(q, k, v, causal, scale):
    Nq, Nk = q.shape[2], k.shape[2]
    mask = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq) if causal else None
    return torch.nn.functional.scaled_dot_product_attention(
        _wide(q), _wide(k), _wide(v), attn_mask=mask, scale=scale).numpy()


def _lse_scipy_qk(q, k, causal, scale):
    s = scale * np.einsum("bhid,bhjd->bhij", _wide(q).numpy(), _wide(k).numpy())
    if causal:
        Nq, Nk = s.shape[-2:]
        s = np.where(np.tril(np.ones((Nq, Nk), dtype=bool), k=Nk - Nq), s, -np.inf)
    return scipy.special.logsumexp(s, axis=-1)


@pytest.mark.parametrize("Nq,Nk,d,causal", [
    (1, 1, 64, True), (1, 300, 64, True), (1, 300, 128, False), (4, 129, 128, True),
    (17, 1000, 64, True), (64, 65, 128, True), (100, 333, 64, False)])
def test_fewer_queries_match_sdpa_with_explicit_mask(Nq, Nk, d, causal):
    q = inputs.make_qkv(2, 2, Nq, d, seed=400 + Nq)[0]
    _, k, v = inputs.make_qkv(2, 2, Nk, d, seed=401 + Nk)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, causal, scale)
    np.testing.assert_allclose(o, _sdpa64_mask(q, k, v, causal, scale), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _lse_scipy_qk(q, k, causal, scale), rtol=0, atol=1e-12)


def test_decode_rows_are_the_last_rows_of_the_full_causal_problem():
    # queries at the last Nq positions see exactly what those rows of the full
    # (Nk x Nk) causal problem see
    Nk, Nq, d = 257, 9, 128
    q, k, v = inputs.make_qkv(1, 3, Nk, d, seed=402)
    o_full, lse_full = oracle.attention(q, k, v, True, 0.0883)
    o, lse = oracle.attention(q[:, :, Nk - Nq:].contiguous(), k, v, True, 0.0883)
    assert np.array_equal(o, o_full[:, :, Nk - Nq:])
    assert np.array_equal(lse, lse_full[:, :, Nk - Nq:])


def test_single_causal_query_sees_every_key():
    q = inputs.make_qkv(1, 2, 1, 64, seed=403)[0]
    _, k, v = inputs.make_qkv(1, 2, 500, 64, seed=404)
    a = oracle.attention(q, k, v, True, 0.125)
    b = oracle.attention(q, k, v, False, 0.125)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_more_queries_than_keys_under_the_causal_mask():
    q = inputs.make_qkv(1, 1, 10, 64, seed=405)[0]
    _, k, v = inputs.make_qkv(1, 1, 9, 64, seed=406)
    with pytest.raises(RuntimeError):
        oracle.attention(q, k, v, True, 0.1)
    oracle.attention(q, k, v, False, 0.1)  # fine without the mask
