"""The seeded input generator: determinism, rounding, shapes and row subsets."""

import torch

from exact_io_aware_27_amd import inputs


def test_same_seed_same_bits_and_order_q_k_v():
    a = inputs.make_qkv(1, 2, 33, 64, seed=5)
    b = inputs.make_qkv(1, 2, 33, 64, seed=5)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 2, 33, 64)
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    g = torch.Generator().manual_seed(5)
    q32 = torch.randn((1, 2, 33, 64), generator=g)
    assert torch.equal(a[0], q32.to(torch.bfloat16))
    c = inputs.make_qkv(1, 2, 33, 64, seed=6)
    assert not torch.equal(a[0], c[0])


def test_bf16_conversion_rounds_to_nearest_even():
    one = 1.0
    half_ulp = 2.0 ** -8  # bf16 has 7 stored mantissa bits: ulp(1) = 2^-7
    x = torch.tensor([one + half_ulp, one + 3 * half_ulp, one + 1.5 * half_ulp])
    y = x.to(torch.bfloat16).float()
    assert y.tolist() == [1.0, 1.0 + 4 * half_ulp, 1.0 + 2 * half_ulp]


def test_sigma_scales_spread():
    q, _, v = inputs.make_qkv(1, 1, 4096, 128, seed=4, sigma_qk=4.0)
    assert 3.8 < q.float().std().item() < 4.2
    assert 0.95 < v.float().std().item() < 1.05


def test_row_subsets_sorted_distinct_forced_and_seeded():
    w = inputs.WORKLOADS[4]
    r = inputs.row_subsets(w)
    assert r.shape == (w.B * w.H, w.rows_checked)
    for row in r:
        assert torch.equal(row, torch.sort(row).values)
        assert len(set(row.tolist())) == row.numel()
        assert row[0].item() == 0 and row[-1].item() == w.N - 1
    assert torch.equal(r, inputs.row_subsets(w))
    assert not torch.equal(r[0], r[1])
    assert torch.equal(inputs.row_subset(10, 20, 1, 0), torch.arange(10))


def test_workload_table():
    names = [w.name for w in inputs.WORKLOADS]
    assert len(names) == 5 and inputs.HEADLINE.N == 8192 and inputs.HEADLINE.causal
    assert inputs.HEADLINE.flops == 4 * 2 * 32 * 8192 ** 2 * 128 / 2
    assert inputs.WORKLOADS[3].sigma_qk == 4.0 and not inputs.WORKLOADS[3].causal


def test_make_q_kv_matches_make_qkv_when_lengths_agree():
    a = inputs.make_q_kv(2, 3, 17, 17, 64, seed=9)
    b = inputs.make_qkv(2, 3, 17, 64, seed=9)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_make_q_kv_shapes_and_determinism():
    q, k, v = inputs.make_q_kv(1, 2, 3, 50, 128, seed=10)
    assert q.shape == (1, 2, 3, 128) and k.shape == v.shape == (1, 2, 50, 128)
    q2, k2, v2 = inputs.make_q_kv(1, 2, 3, 50, 128, seed=10)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)


def test_split_workload_visible_pairs_by_brute_force():
    for w in [inputs.SplitWorkload("t", 1, 1, 5, 9, 64, True, 2, 1, 0),
              inputs.SplitWorkload("t", 1, 1, 5, 9, 64, False, 2, 1, 0),
              inputs.SplitWorkload("t", 1, 1, 7, 7, 64, True, 2, 1, 0)]:
        off = w.Nk - w.Nq
        n = sum(1 for i in range(w.Nq) for j in range(w.Nk) if (not w.causal) or j <= i + off)
        assert w.visible_pairs == n
    d = {w.name: w for w in inputs.SPLITKV_WORKLOADS}["decode_64k"]
    assert d.kv_bytes == 2 * 2 * 4 * 32 * 65536 * 128 and d.visible_pairs == 65536
