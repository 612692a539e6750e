"""The pages' tiled recurrence and merge identity equal the plain definition.

This pins the reading of the online-softmax iteration (scale from the
attention equation, initial m = -inf / l = 0 / O = 0, final division by l)
that the HIP kernel implements, against the C oracle's definition.
"""

import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import online
from exact_io_aware_27_amd import inputs


def _wide(x):
    return x.double().numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("blocks", [(1, 1), (7, 7), (64, 64), (None, None), (128, 32), (5, 64)])
def test_tiled_recurrence_equals_definition(causal, blocks):
    N, d = 200, 64
    q, k, v = inputs.make_qkv(1, 1, N, d, seed=21, sigma_qk=2.0)
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = oracle.attention(q, k, v, causal, scale)
    o, lse = online.online_attention(_wide(q)[0, 0], _wide(k)[0, 0], _wide(v)[0, 0], causal, scale,
                                     block_q=blocks[0], block_kv=blocks[1])
    np.testing.assert_allclose(o, o_ref[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref[0, 0], rtol=0, atol=1e-12)


def test_merge_stats_matches_direct_max_and_sum():
    rng = np.random.default_rng(22)
    for _ in range(20):
        x1 = rng.normal(size=rng.integers(1, 9)) * 30
        x2 = rng.normal(size=rng.integers(1, 9)) * 30
        m1, m2 = x1.max(), x2.max()
        l1, l2 = np.exp(x1 - m1).sum(), np.exp(x2 - m2).sum()
        m, l, a1, a2 = online.merge_stats(m1, l1, m2, l2)
        x = np.concatenate([x1, x2])
        assert m == x.max()
        assert abs(l - np.exp(x - x.max()).sum()) <= 1e-12 * l
        # softmax(x) = f(x) / l(x) with f = [a1 f1, a2 f2]
        f = np.concatenate([a1 * np.exp(x1 - m1), a2 * np.exp(x2 - m2)])
        np.testing.assert_allclose(f / l, scipy.special.softmax(x), rtol=1e-12, atol=1e-300)


def test_merge_partials_of_disjoint_key_sets():
    """Partials over two key sets merge to the attention over their union."""
    rng = np.random.default_rng(23)
    s = rng.normal(size=(5, 30)) * 8
    vv = rng.normal(size=(30, 16))

    def part(cols):
        p = scipy.special.softmax(s[:, cols], axis=1)
        return p @ vv[cols], scipy.special.logsumexp(s[:, cols], axis=1)

    o1, l1 = part(np.arange(0, 11))
    o2, l2 = part(np.arange(11, 30))
    o, lse = online.merge_partials(o1, l1, o2, l2)
    np.testing.assert_allclose(o, scipy.special.softmax(s, axis=1) @ vv, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=1), rtol=0, atol=1e-12)
