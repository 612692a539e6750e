"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws random bf16 tensors
and random row subsets.  It is the one module that both the HIP path's
callers and the oracle's callers use, so that both see the same bits.

Recipe (one CPU torch.Generator per workload, seeded with the workload's
seed): draw Q, then K, then V, each as float32 standard normals times sigma,
then round to bfloat16 with round-to-nearest-even (torch's ``.to``).
"""

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    sigma_qk: float
    sigma_v: float
    seed: int
    rows_checked: int  # query rows per (batch, head) the oracle checks; 0 = all

    @property
    def scale(self):
        return 1.0 / (self.d ** 0.5)

    @property
    def flops(self):
        """Counted work 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def describe(self):
        return "%s B=%d H=%d N=%d d=%d %s" % (
            self.name, self.B, self.H, self.N, self.d, "causal" if self.causal else "non-causal")


# The five workloads: a tiny non-causal case, a GPT-2-small-shaped causal case,
# the long-context causal case (the headline), a non-causal long case with
# large logits (Q, K ~ N(0, 4^2)), and a very long causal case.
WORKLOADS = [
    Workload("tiny", 1, 2, 256, 64, False, 1.0, 1.0, 1, 0),
    Workload("gpt2_small", 8, 12, 1024, 64, True, 1.0, 1.0, 2, 0),
    Workload("long_causal", 2, 32, 8192, 128, True, 1.0, 1.0, 3, 0),
    Workload("large_logits", 1, 16, 16384, 128, False, 4.0, 1.0, 4, 2048),
    Workload("very_long_causal", 1, 8, 65536, 128, True, 1.0, 1.0, 5, 1024),
]
HEADLINE = WORKLOADS[2]


@dataclass(frozen=True)
class SplitWorkload:
    """A split-KV workload: Nq queries against Nk keys, cut into `splits` key
    ranges (queries at the last Nq positions under the causal mask)."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    splits: int
    seed: int
    rows_checked: int  # query rows per (batch, head) the oracle checks; 0 = all

    @property
    def scale(self):
        return 1.0 / (self.d ** 0.5)

    @property
    def visible_pairs(self):
        """Visible (query, key) pairs per head."""
        if not self.causal:
            return self.Nq * self.Nk
        off = self.Nk - self.Nq  # query i sees keys 0 .. i + off
        return self.Nq * (off + 1) + self.Nq * (self.Nq - 1) // 2

    @property
    def flops(self):
        return 4.0 * self.B * self.H * self.visible_pairs * self.d

    @property
    def kv_bytes(self):
        """K and V read once (bf16)."""
        return 2 * 2 * self.B * self.H * self.Nk * self.d

    def describe(self, splits=None):
        return "%s B=%d H=%d Nq=%d Nk=%d d=%d %s splits=%d" % (
            self.name, self.B, self.H, self.Nq, self.Nk, self.d,
            "causal" if self.causal else "non-causal", self.splits if splits is None else splits)


# Split-KV workloads: decoding (one new query per head against 64K cached
# keys; memory-bound) and one long head (too few query tiles to fill the
# chip without splitting the keys).
SPLITKV_WORKLOADS = [
    SplitWorkload("decode_64k", 4, 32, 1, 65536, 128, True, 4, 11, 0),
    SplitWorkload("one_head_16k", 1, 1, 16384, 16384, 128, False, 4, 12, 256),
]


def make_q_kv(B, H, Nq, Nk, d, seed, sigma_qk=1.0, sigma_v=1.0):
    """Q [B, H, Nq, d], then K and V [B, H, Nk, d], CPU bfloat16, one generator."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = (torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32) * sigma_qk).to(torch.bfloat16)
    k = (torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32) * sigma_qk).to(torch.bfloat16)
    v = (torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32) * sigma_v).to(torch.bfloat16)
    return q, k, v


def make_grad_out(B, H, Nq, d, seed, sigma=1.0):
    """Upstream gradient dO [B, H, Nq, d] for the backward pass, CPU bfloat16,
    standard normal times sigma from its own generator."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return (torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32) * sigma).to(torch.bfloat16)


def make_signs(d, seed):
    """The random signs of incoherent processing: d values +-1 (float32)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return (torch.randint(0, 2, (d,), generator=g) * 2 - 1).to(torch.float32)


def make_qkv_outliers(B, H, N, d, seed, frac=1e-3, outlier_sigma=10.0):
    """Q, K, V as make_qkv (standard normal), then a fraction `frac` of the
    entries of each, at seeded positions, replaced by normals of standard
    deviation outlier_sigma: the outlier-heavy input on which per-tensor FP8
    loses accuracy.  CPU bfloat16."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = []
    for _ in range(3):
        x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
        hit = torch.rand((B, H, N, d), generator=g) < frac
        x = torch.where(hit, torch.randn((B, H, N, d), generator=g) * outlier_sigma, x)
        out.append(x.to(torch.bfloat16))
    return tuple(out)


def make_kv_on_device(B, H, Nk, d, seed, device):
    """K and V [B, H, Nk, d] drawn on `device` (standard normal, bfloat16) by a
    seeded generator there: for the largest key counts, whose fp32 draws on
    the host would take minutes and tens of GB."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    k = torch.randn((B, H, Nk, d), generator=g, device=device, dtype=torch.bfloat16)
    v = torch.randn((B, H, Nk, d), generator=g, device=device, dtype=torch.bfloat16)
    return k, v


def make_qkv(B, H, N, d, seed, sigma_qk=1.0, sigma_v=1.0):
    """Q, K, V as CPU bfloat16 tensors [B, H, N, d], drawn in that order."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk).to(torch.bfloat16)
    k = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk).to(torch.bfloat16)
    v = (torch.randn(shape, generator=g, dtype=torch.float32) * sigma_v).to(torch.bfloat16)
    return q, k, v


def workload_qkv(w):
    return make_qkv(w.B, w.H, w.N, w.d, w.seed, w.sigma_qk, w.sigma_v)


def row_subset(N, R, seed, bh, force=()):
    """A sorted, seeded subset of R distinct query rows of [0, N) for head bh.

    The generator is seeded with seed*1000003 + bh.  Rows listed in ``force``
    replace the last drawn rows that are not already forced, so they are
    always present.  R >= N returns every row.
    """
    if R >= N:
        return torch.arange(N, dtype=torch.int64)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) * 1000003 + int(bh))
    rows = torch.randperm(N, generator=g)[:R].tolist()
    forced = [f for f in dict.fromkeys(force) if 0 <= f < N]
    rest = [r for r in rows if r not in forced]
    rows = forced + rest[:R - len(forced)]
    return torch.tensor(sorted(rows), dtype=torch.int64)


def row_subsets(w, R=None, force_ends=True):
    """Rows per (batch, head) for workload w: int64 tensor [B*H, R]."""
    R = R if R is not None else (w.rows_checked or w.N)
    force = (0, w.N - 1) if force_ends else ()
    return torch.stack([row_subset(w.N, R, w.seed, bh, force) for bh in range(w.B * w.H)])
