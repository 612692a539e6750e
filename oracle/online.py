"""The pages' tiled (online-softmax) recurrence and two-block merge, in NumPy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The plain definition lives in attn_oracle.c.  This module writes out the
*algorithm* the pages give for reaching the same result block by block, so a
test can show that the reading of that algorithm used by the HIP kernel is
the definition, up to rounding order:

- "FlashAttention evolution" (letsgetai.github.io), section on the core
  mechanism: the two-block merge equations for m, l and f, and the final
  division by l once at the end.
- "FlashAttention" concept page (compassingai.com), section 3, the online
  softmax iteration: per key/value block, a new row max, exponentials against
  it, the old sum and old output rescaled by exp(m_old - m_new), then the new
  block's contribution added.

Readings where the pages are silent (also listed in the design doc): the iteration
as printed omits the scale (taken from the attention equation) and the final
division by l (taken from the merge section); initial values are m = -inf,
l = 0, O = 0; f(x) in the merge equation is exp(x - m(x)) elementwise, so
l(x) = sum f(x).

Parity: pinned against the C definition (tests/test_online.py) for block
sizes 1, 7, 64 and N, and against closed forms.
"""

import numpy as np


def merge_stats(m1, l1, m2, l2):
    """Two-block merge of the softmax statistics (the pages' merge equation).

    m = max(m1, m2);  l = exp(m1 - m) l1 + exp(m2 - m) l2.
    Returns (m, l, a1, a2) with a_g = exp(m_g - m), the factors the merged
    f = [a1 f1, a2 f2] applies to each block's unnormalised weights.
    """
    m = np.maximum(m1, m2)
    a1 = np.exp(m1 - m)
    a2 = np.exp(m2 - m)
    return m, a1 * l1 + a2 * l2, a1, a2


def merge_partials(o1, lse1, o2, lse2):
    """Merge two normalised partial attentions over disjoint key sets.

    A partial over key set K_g carries O_g = sum_j f_j v_j / l_g and
    LSE_g = m_g + ln l_g.  Splitting LSE_g back into (m_g, l_g) = (LSE_g, 1)
    is exact for the merge, because the merge equation only ever uses
    exp(m_g) l_g.  Applying merge_stats to those statistics gives
    LSE = m + ln l and O = (a1 l1 O_1 + a2 l2 O_2) / l.
    Shapes: o_g [..., d], lse_g [...].  fp64 in, fp64 out.
    """
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    m, l, a1, a2 = merge_stats(lse1, 1.0, lse2, 1.0)
    o = (a1[..., None] * np.asarray(o1, dtype=np.float64) +
         a2[..., None] * np.asarray(o2, dtype=np.float64)) / l[..., None]
    return o, m + np.log(l)


def online_attention(q, k, v, causal, scale, block_q=None, block_kv=None):
    """Tiled exact attention for ONE head in fp64, in the pages' loop order.

    q, k, v: float64 arrays [N, d] (bf16 values already widened).
    Outer loop over query blocks, inner loop over key/value blocks (the
    FlashAttention-2 loop order); within each, the online-softmax update.
    Causal: key j is visible to query i iff j <= i; masked logits are -inf.
    Returns (o [N, d], lse [N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    bq = block_q or N
    bkv = block_kv or N
    o_all = np.empty((N, d))
    lse_all = np.empty(N)
    for q0 in range(0, N, bq):
        qi = q[q0:q0 + bq]
        rows = np.arange(q0, q0 + qi.shape[0])
        m = np.full(qi.shape[0], -np.inf)
        l = np.zeros(qi.shape[0])
        acc = np.zeros((qi.shape[0], d))
        for k0 in range(0, N, bkv):
            kj = k[k0:k0 + bkv]
            vj = v[k0:k0 + bkv]
            s = scale * (qi @ kj.T)
            if causal:
                cols = np.arange(k0, k0 + kj.shape[0])
                s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            # A row whose keys so far are all masked keeps m = -inf; its
            # exponentials are all zero, and exp(-inf - -inf) must not be NaN.
            m_use = np.where(np.isneginf(m_new), 0.0, m_new)
            p = np.exp(s - m_use[:, None])
            alpha = np.exp(m - m_use)
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ vj
            m = m_new
        o_all[q0:q0 + qi.shape[0]] = acc / l[:, None]
        lse_all[q0:q0 + qi.shape[0]] = m + np.log(l)
    return o_all, lse_all
