"""The oracle's pins catch plausible slips.

Each mutant is attn_oracle.c with one deliberate mistake, compiled into a
temporary library on the CPU.  The pin suite below (the same kinds of checks
as test_oracle.py: PyTorch float64 SDPA, the golden closed forms, equal keys,
causal row 0) must report at least one failure for every mutant, and none for
the unmodified source.  Every mutant keeps all memory accesses in bounds.
"""

import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import oracle as oracle_impl
from exact_io_aware_27_amd import inputs
import golden_cases

MUTANTS = {
    "dropped_scale": ("S[j] = c->scale * dot;", "S[j] = dot;"),
    "doubled_scale": ("S[j] = c->scale * dot;", "S[j] = 2.0 * c->scale * dot;"),
    "no_max_subtraction": ("P[j] = exp(S[j] - m);", "P[j] = exp(S[j]);"),
    "min_instead_of_max": ("if (S[j] > m)", "if (S[j] < m)"),
    "causal_excludes_diagonal": ("c->causal ? i + (Nk - Nq) + 1 : Nk",
                                 "c->causal ? (i + (Nk - Nq) > 0 ? i + (Nk - Nq) : 1) : Nk"),
    "causal_wrong_direction": ("c->causal ? i + (Nk - Nq) + 1 : Nk", "c->causal ? Nk - i : Nk"),
    "causal_top_left_aligned": ("c->causal ? i + (Nk - Nq) + 1 : Nk", "c->causal ? i + 1 : Nk"),
    "key_head_stride_of_queries": ("const uint16_t *k = c->k + bh * Nk * d;",
                                   "const uint16_t *k = c->k + bh * Nq * d;"),
    "lse_base_two": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "lse_drops_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "value_from_keys": ("o_out[t] += p * widen_bf16(v[j * d + t]);",
                        "o_out[t] += p * widen_bf16(k[j * d + t]);"),
    "query_times_queries": ("dot += qrow[t] * widen_bf16(k[j * d + t]);",
                            "dot += qrow[t] * widen_bf16(q[j * d + t]);"),
    "query_row_zero_only": ("qrow[t] = widen_bf16(q[i * d + t]);", "qrow[t] = widen_bf16(q[t]);"),
    "head_offset_lost": ("const uint16_t *v = c->v + bh * Nk * d;", "const uint16_t *v = c->v;"),
}


def _build(src_text, path):
    with open(path + ".c", "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                           "-o", path, path + ".c", "-lm"])
    return oracle_impl.load_library(path)


def _pin_failures(lib):
    """Run a compact pin suite against `lib`; return the names of failing pins."""
    fails = []

    def check(name, fn):
        try:
            with np.errstate(all="ignore"):
                ok = fn()
        except Exception:
            ok = False
        if not ok:
            fails.append(name)

    def sdpa(N, d, causal):
        q, k, v = inputs.make_qkv(1, 2, N, d, seed=300 + N)
        sc = 1.0 / math.sqrt(d)
        o, _ = oracle.attention(q, k, v, causal, sc, lib=lib, nthreads=2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.double(), k.double(), v.double(), is_causal=causal, scale=sc).numpy()
        return np.allclose(o, ref, rtol=0, atol=1e-12)

    check("sdpa_causal", lambda: sdpa(65, 64, True))
    check("sdpa_noncausal", lambda: sdpa(70, 64, False))

    def sdpa_fewer_queries(Nq, Nk, d, causal):
        # the library routine with an explicit mask: key j visible to query i
        # iff j <= i + (Nk - Nq)
        q = inputs.make_qkv(1, 2, Nq, d, seed=310 + Nq)[0]
        _, k, v = inputs.make_qkv(1, 2, Nk, d, seed=311 + Nk)
        sc = 1.0 / math.sqrt(d)
        o, _ = oracle.attention(q, k, v, causal, sc, lib=lib, nthreads=2)
        mask = None
        if causal:
            mask = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.double(), k.double(), v.double(), attn_mask=mask, scale=sc).numpy()
        return np.allclose(o, ref, rtol=0, atol=1e-12)

    check("sdpa_fewer_queries_causal", lambda: sdpa_fewer_queries(5, 70, 64, True))
    check("sdpa_fewer_queries_noncausal", lambda: sdpa_fewer_queries(3, 41, 64, False))

    for case in golden_cases.load():
        def golden(case=case):
            o, lse = oracle.attention(case["q"], case["k"], case["v"], case["causal"],
                                      case["scale"], lib=lib, nthreads=1)
            return (np.allclose(o[0, 0], case["o"], rtol=0, atol=1e-14) and
                    np.allclose(lse[0, 0], case["lse"], rtol=1e-15, atol=1e-13))
        check("golden_" + case["name"], golden)

    def equal_keys():
        N, d = 40, 64
        q, _, v = inputs.make_qkv(1, 1, N, d, seed=301)
        krow = inputs.make_qkv(1, 1, 1, d, seed=302)[1]
        k = krow.expand(1, 1, N, d).contiguous()
        o, lse = oracle.attention(q, k, v, True, 0.125, lib=lib, nthreads=1)
        s = 0.125 * (q.double()[0, 0] @ krow.double()[0, 0, 0]).numpy()
        vv = v.double()[0, 0].numpy()
        return all(np.allclose(o[0, 0, i], vv[:i + 1].mean(0), rtol=0, atol=1e-13) and
                   abs(lse[0, 0, i] - s[i] - math.log(i + 1)) < 1e-12 for i in range(N))
    check("equal_keys", equal_keys)
    return fails


@pytest.fixture(scope="module")
def source():
    with open(os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")) as f:
        return f.read()


def test_unmodified_source_passes_the_suite(source, tmp_path):
    lib = _build(source, str(tmp_path / "liboracle_clean.so"))
    assert _pin_failures(lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, "mutation site not found: %r" % old
    lib = _build(source.replace(old, new), str(tmp_path / ("liboracle_%s.so" % name)))
    assert _pin_failures(lib), "no pin caught mutant %s" % name
