"""FP8 attention: block quantization with incoherent processing, and the
exact attention the FP8 path approximates (NumPy, fp64 unless stated).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages describe FlashAttention-3's FP8 mode only in outline: FP8 tensor
cores, block quantization (one scale per block of the tensor instead of one
per tensor) and incoherent processing, which multiplies Q and K by a random
orthogonal matrix so that outliers spread over the head dimension before
quantization; the product QK^T is unchanged in exact arithmetic ("FlashAttention
evolution", letsgetai.github.io, FlashAttention-3 section and its results;
"FlashAttention 1-4 evolution cheat sheet", argus-lessons, FlashAttention-3
section).  The readings taken here where they are silent:

  * FP8 is the OCP E4M3 format (largest finite 448, smallest subnormal 2^-9),
    round to nearest even.
  * A block is 64 consecutive rows of one head (all d columns); its scale is
    the power of two 2^E with E the smallest integer such that the block's
    largest magnitude is at most 448 * 2^E (so no value saturates).  An
    all-zero block takes E = 0.
  * The orthogonal matrix is M = diag(s) H / sqrt(d): random signs s, then the
    Sylvester-ordered Hadamard matrix H.  The rotation is applied to Q and K
    without the 1/sqrt(d) (x -> (x * s) H, exact in the sense that H has +-1
    entries), and the factor 1/d = (1/sqrt(d))^2 moves into the softmax scale,
    which keeps every rounding of the rotation inside one fp32 butterfly
    network: the fast Walsh-Hadamard transform with strides 1, 2, 4, ...,
    d/2, each stage (a, b) -> (a + b, a - b) in fp32.  The rotated values are
    quantized, so the rotation's fp32 roundings decide FP8 codes; they are
    taken in fp32 here, in this order, as in the kernel.
  * V is quantized in blocks of 64 keys without rotation.
  * Q alone is multiplied, after its rotation and before it is quantized, by
    c = scale * log2(e) in fp32 (one fp32 product of the fp32 scale and
    log2(e) rounded to fp32, then 1/d when rotated, exact), so that the
    product of the quantized operands is the logits in log2 units.  The pages
    do not say where the softmax scale enters the FP8 products; here it rides
    with Q's quantization, whose relative rounding error does not depend on
    the magnitude of what it rounds.

Parity unpinned: the size of the pages' FP8 error reduction (2.6x against
per-tensor FP8).  The pages give no input distribution for it; on the
outlier-heavy synthetic input of the tests the emulation here shows the
direction of the gain (1.8x), not its size.

Functions:
  e4m3_round       the E4M3 grid (RNE) on values of magnitude <= 448
  hadamard         the Sylvester Hadamard matrix (+-1 entries)
  fwht_f32         the fp32 butterfly network above
  block_quantize   per-64-row power-of-two scales and E4M3 values
  tensor_quantize  one power-of-two scale for a whole tensor (the baseline
                   the pages compare block quantization against)
  prepare_fp8      Q, K (rotated or not) and V of a [B, H, N, d] problem,
                   quantized, dequantized, with the exponents
  attention_fp64   exact attention on given (dequantized) inputs, with the
                   expected size of the error that rounding P to E4M3 adds
  attention_fp8    the whole FP8 method on the CPU: attention of the
                   dequantized inputs with P (relative to its row max)
                   rounded to E4M3 before P V, O divided by the unrounded sum
"""

import numpy as np

E4M3_MAX = 448.0
BLOCK = 64


def e4m3_round(x):
    """Round float64 values to the nearest E4M3 value (ties to even).

    |x| must be at most 448: a block scale is chosen so that nothing
    saturates, so a larger input is a caller error.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E4M3_MAX) or not np.all(np.isfinite(x)):
        raise ValueError("e4m3_round: input outside [-448, 448]")
    _, e = np.frexp(a)  # a = f * 2^e, f in [0.5, 1): floor(log2 a) = e - 1
    # three fraction bits: quantum 2^(floor(log2 a) - 3); below 2^-6 the
    # subnormal quantum 2^-9
    quantum = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    return np.round(x / quantum) * quantum  # x / quantum is exact; np.round is half-even


def hadamard(d):
    """The d x d Sylvester Hadamard matrix: H_1 = [1], H_2n = [[H, H], [H, -H]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32(x):
    """x (float32 [..., d]) times the Sylvester Hadamard matrix, by butterfly
    stages of stride 1, 2, ..., d/2, each (a, b) -> (a + b, a - b) in fp32."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        z = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return y


def block_exponent(amax):
    """Smallest integer E with amax <= 448 * 2^E (0 for amax == 0), within
    the E8M0 range [-127, 127]."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    _, e = np.frexp(amax / E4M3_MAX)
    E = int(e)  # amax / 448 < 2^e, but the division rounded: check exactly
    while E > -127 and amax <= E4M3_MAX * 2.0 ** (E - 1):
        E -= 1
    while amax > E4M3_MAX * 2.0 ** E:
        E += 1
    return max(-127, min(127, E))


def block_quantize(x, block=BLOCK):
    """x: float32/float64 [..., R, d].  Rows are cut into blocks of `block`
    (the last one ragged); each block gets the exponent of its largest
    magnitude.  Returns (codes, exps): codes float64 on the E4M3 grid (the
    value stored), exps int [..., ceil(R / block)]; x ~= codes * 2^exps."""
    x = np.asarray(x, dtype=np.float64)
    R = x.shape[-2]
    nb = (R + block - 1) // block
    codes = np.empty_like(x)
    exps = np.empty(x.shape[:-2] + (nb,), dtype=np.int64)
    for idx in np.ndindex(*x.shape[:-2]):
        for b in range(nb):
            blk = x[idx][b * block:(b + 1) * block]
            E = block_exponent(np.abs(blk).max() if blk.size else 0.0)
            exps[idx + (b,)] = E
            codes[idx][b * block:(b + 1) * block] = e4m3_round(blk / 2.0 ** E)
    return codes, exps


def tensor_quantize(x):
    """One exponent for all of x (per-tensor FP8).  Returns (codes, E)."""
    x = np.asarray(x, dtype=np.float64)
    E = block_exponent(np.abs(x).max() if x.size else 0.0)
    return e4m3_round(x / 2.0 ** E), E


def dequantize(codes, exps, block=BLOCK):
    """codes [..., R, d] times 2^exps per block of rows."""
    R = codes.shape[-2]
    scale = np.repeat(np.ldexp(1.0, np.asarray(exps)), block, axis=-1)[..., :R]
    return codes * scale[..., None]


def prepare_fp8(q, k, v, signs=None, per_tensor=False, scale=None):
    """Quantize bf16/float q, k, v [B, H, N, d] the way the FP8 path does.

    signs: None (no incoherent processing) or +-1 float array [d]: Q and K are
    rotated by fwht_f32(x * signs) first (their product gains the factor d).
    per_tensor: one exponent per tensor instead of per 64-row block.
    scale: None, or the softmax scale: Q (after the rotation) is then
    multiplied in fp32 by c = fp32(scale) * fp32(log2 e), times 1/d when
    rotated, before it is quantized.
    Returns a dict of dequantized float64 tensors 'q', 'k', 'v', the codes
    'qc', 'kc', 'vc', the exponents 'qe', 'ke', 've', 'qk_factor' (the
    factor the product QK^T gained: d with rotation, else 1) and 'qk_mul'
    (with scale: ln 2, which turns the product of the dequantized operands
    into natural-log logits; else None).
    """
    def f32(x):
        import torch
        return x.float().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float32)

    qf, kf, vf = f32(q), f32(k), f32(v)
    d = qf.shape[-1]
    if signs is not None:
        s = np.asarray(signs, dtype=np.float32)
        qf = fwht_f32(qf * s)
        kf = fwht_f32(kf * s)
    if scale is not None:
        c = np.float32(scale) * np.float32(np.log2(np.e))
        if signs is not None:
            c = c * np.float32(1.0 / d)
        qf = (qf * c).astype(np.float32)
    out = {"qk_factor": float(d) if signs is not None else 1.0,
           "qk_mul": float(np.log(2.0)) if scale is not None else None}
    for name, x in (("q", qf), ("k", kf), ("v", vf)):
        if per_tensor:
            c, E = tensor_quantize(x)
            out[name + "c"], out[name + "e"] = c, E
            out[name] = c * 2.0 ** E
        else:
            c, e = block_quantize(x)
            out[name + "c"], out[name + "e"] = c, e
            out[name] = dequantize(c, e)
    return out


def attention_fp64(q, k, v, causal, scale, p_rounding=False):
    """Exact attention of float64 q [B, H, Nq, d] against k, v [B, H, Nk, d]
    (causal: query i sees key j iff j <= i + Nk - Nq).

    Returns (o, lse) and, with p_rounding, sigma [B, H, Nq, d]: the standard
    deviation that rounding each P_ij to E4M3 before P V (O divided by the
    sum of the unrounded weights) adds to O, for rounding errors uniform over
    half a quantum: 2^-4 relative for P >= 2^-6 (P relative to the row max),
    2^-10 absolute below.  O' - O = sum_j (P'_j - P_j) v_j / sum_j P_j.
    """
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    Nq, Nk = q.shape[2], k.shape[2]
    if causal:
        mask = np.tril(np.ones((Nq, Nk), dtype=bool), Nk - Nq)
        s = np.where(mask, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=-1, keepdims=True)
    o = np.einsum("bhij,bhjd->bhid", p, v) / l
    lse = (m + np.log(l))[..., 0]
    if not p_rounding:
        return o, lse
    err = np.where(p >= 2.0 ** -6, p * 2.0 ** -4, 2.0 ** -10) / np.sqrt(3.0)
    err = np.where(p > 0, err, 0.0)
    sigma = np.sqrt(np.einsum("bhij,bhjd->bhid", err ** 2, v * v)) / l
    return o, lse, sigma


def attention_fp8(prep, causal, scale=None):
    """FP8 attention of a prepare_fp8() result: S from the dequantized Q and
    K (times qk_mul when Q carries the scale, else scale / qk_factor, which
    undoes the rotation's factor d), P = exp(S - max) rounded to E4M3,
    O = P' V / sum P, LSE from the unrounded sum.  Returns (o, lse) float64."""
    q, k, v = prep["q"], prep["k"], prep["v"]
    mul = prep["qk_mul"] if prep.get("qk_mul") is not None else scale / prep["qk_factor"]
    s = mul * np.einsum("bhid,bhjd->bhij", q, k)
    Nq, Nk = q.shape[2], k.shape[2]
    if causal:
        s = np.where(np.tril(np.ones((Nq, Nk), dtype=bool), Nk - Nq), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=-1, keepdims=True)
    o = np.einsum("bhij,bhjd->bhid", e4m3_round(p), v) / l
    return o, (m + np.log(l))[..., 0]
