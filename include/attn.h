/*
 * attn.h -- C ABI of libattn.so: exact, fused attention forward pass (and
 * its gradients) on AMD MI355X (gfx950).
 *
 * What the call computes, for every batch b and head h:
 *
 *   O   = softmax(scale * Q K^T) V                 (bf16 out, fp32 arithmetic)
 *   LSE = ln( sum_j exp(scale * q_i . k_j) )       (fp32 out, one per query row)
 *
 * This is the attention equation of "FlashAttention evolution"
 * (letsgetai.github.io), section on why attention is slow, with the scale an
 * explicit argument (that equation uses 1/sqrt(d)).  The result is reached
 * with the tiled online softmax of the same page's core-mechanism section
 * (running max m and running sum l, merged block by block with the two-block
 * merge equation, divided by l once at the end) and with the FlashAttention-2
 * loop order and sequence parallelism of "FlashAttention 1-4 evolution cheat
 * sheet" (argus-lessons), FlashAttention-2 section.  The N x N score and
 * probability matrices never leave the chip.  Results equal the definition up
 * to floating-point accumulation order, not bit for bit (the numerical
 * equivalence paragraph of the "FlashAttention" concept page,
 * compassingai.com, section 3).
 *
 * LSE is the natural-log logsumexp of the scaled, masked logits, i.e. the
 * saved softmax statistics m + ln(l) that a recomputing backward pass needs
 * ("FlashAttention evolution", recomputation paragraph).
 *
 * Causal mask: key j is visible to query i iff j <= i + (Nk - Nq); with as
 * many queries as keys (attn_fwd) that is j <= i.  Fewer queries than keys
 * (attn_fwd_splitkv) are the last Nq positions of the sequence, as when
 * decoding with the keys and values of earlier tokens kept.  Masked logits
 * take no part in the max, the sum or the output.
 */
#ifndef EXACT_IO_AWARE_ATTN_H
#define EXACT_IO_AWARE_ATTN_H

#include <stdint.h>

#if defined(__GNUC__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by attn_fwd(), attn_fwd_splitkv() and attn_bwd(). */
enum attn_status {
    ATTN_OK = 0,
    ATTN_NULL_PTR = 1,      /* q, k, v or o is NULL (and the problem is not empty) */
    ATTN_BAD_SHAPE = 2,     /* B, H, N (Nq, Nk) negative; N * d >= 2^31; a byte size or
                               the workgroup count overflows; split-KV only: Nk == 0
                               with queries, causal Nq > Nk, num_splits < 1 */
    ATTN_UNSUPPORTED_D = 3, /* d is neither 64 nor 128 */
    ATTN_BAD_SCALE = 4,     /* scale is NaN or infinite */
    ATTN_MISALIGNED = 5,    /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
    ATTN_ALIAS = 6,         /* o or lse overlaps q, k or v, or o overlaps lse */
    ATTN_HIP = 7,           /* the kernel launch failed; see attn_last_hip_error() */
    ATTN_BAD_WORKSPACE = 8, /* attn_fwd_splitkv, attn_bwd: workspace NULL, not 16-byte
                               aligned, smaller than the *_workspace_bytes() size, or
                               overlapping a tensor of the call */
    ATTN_BAD_ARGUMENT = 9,  /* attn_fp8_quantize: signs given with the transposed layout */
    ATTN_SCRATCH_TOO_SMALL = 10 /* attn_fwd_splitkv_noalloc: the call needs more than
                                   attn_noalloc_scratch_bytes() of scratch */
};

/*
 * attn_fwd -- O = softmax(scale * Q K^T) V and LSE, for all B*H heads.
 *
 * q, k, v  device pointers, bf16, contiguous [B][H][N][d] (d fastest).
 * o        device pointer, bf16, contiguous [B][H][N][d]; fully overwritten.
 * lse      device pointer, fp32, contiguous [B][H][N], natural log; fully
 *          overwritten.  NULL: LSE is not written.
 * B, H, N  batch, heads, sequence length (queries == keys == N).  Any of them
 *          0 makes the call an immediate no-op returning ATTN_OK.  N need not
 *          be a multiple of any tile size.
 * d        head dimension: 64 or 128.
 * causal   0: every key visible;  nonzero: key j visible to query i iff j <= i.
 * scale    multiplies q . k before the softmax (usually 1/sqrt(d)); finite.
 * stream   a hipStream_t passed as void*; NULL is the null (default) stream.
 *
 * Ownership: the caller owns every buffer.  The library allocates no device
 * or host memory, keeps no state between calls and is reentrant; calls on
 * different streams may run concurrently.
 * Asynchrony: the call enqueues one kernel on `stream` and returns without
 * synchronising.  Faults inside the kernel surface at the caller's next
 * synchronisation, not here.
 * Errors: arguments are checked in this order, before any HIP runtime call,
 * so every code but ATTN_HIP is returned without touching a GPU:
 * BAD_SHAPE, UNSUPPORTED_D, BAD_SCALE, (empty -> OK), NULL_PTR, MISALIGNED,
 * ALIAS.  No C++ exception crosses this interface.
 */
ATTN_API int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             int64_t B, int64_t H, int64_t N, int64_t d, int causal,
             float scale, void *stream);

/*
 * attn_fwd_splitkv -- the same result with the keys cut into ranges that
 * separate workgroups process in parallel, then merged: FlashDecoding's
 * parallelism over the key sequence ("FlashAttention" concept page,
 * compassingai.com, section 5, evolution timeline) with the two-block merge
 * equation of "FlashAttention evolution" (letsgetai.github.io, core-mechanism
 * section) applied to the ranges: LSE = log sum_s exp(LSE_s) and
 * O = sum_s exp(LSE_s - LSE) O_s.  It keeps the chip busy when B * H * Nq is
 * small next to Nk (few heads, or decoding with Nq = 1).
 *
 * q, o     bf16, contiguous [B][H][Nq][d];  lse: fp32 [B][H][Nq] or NULL.
 * k, v     bf16, contiguous [B][H][Nk][d].
 * Nq, Nk   queries and keys per head, Nk >= 1; under the causal mask
 *          Nq <= Nk (the queries are the last Nq positions).  Nq == 0, B == 0
 *          or H == 0 is an immediate no-op.
 * num_splits  requested key ranges, >= 1.  A range holds
 *          ceil(Nk / num_splits) keys rounded up to a multiple of 128, so
 *          fewer ranges may be used.  When one range results (num_splits
 *          == 1, or Nk <= 128), one pass writes o and lse directly and the
 *          workspace is not touched (and may be NULL).
 * workspace, workspace_bytes  device scratch for the per-range fp32 O and
 *          LSE, at least attn_fwd_splitkv_workspace_bytes(B, H, Nq, d,
 *          num_splits) bytes, 16-byte aligned, owned by the caller.  Its
 *          contents on entry are ignored and on return are undefined; two
 *          calls in flight must not share one workspace.
 * Other arguments, ownership and asynchrony as attn_fwd (two kernels are
 * enqueued when more than one range is used).  Errors are checked in the
 * order of attn_fwd, with num_splits < 1 and causal Nq > Nk as BAD_SHAPE,
 * then BAD_WORKSPACE after ALIAS.
 */
ATTN_API int attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                     int causal, float scale, int64_t num_splits,
                     void *workspace, int64_t workspace_bytes, void *stream);

/*
 * attn_fwd_splitkv_noalloc -- attn_fwd_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and result, without
 * the workspace arguments.  The per-range partials go to scratch memory the
 * library holds: one file-scope device array of attn_noalloc_scratch_bytes()
 * bytes on each GPU the library runs on, kept until the process ends.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Its first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress, with that device current), so call it with
 * the current device set to the one `stream` belongs to.
 *
 * Every call on one GPU shares that GPU's array, whose contents are left as
 * the last call wrote them: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  Every
 * element a call reads back was written earlier in the same call, so nothing
 * needs clearing between calls.
 *
 * Errors: as attn_fwd_splitkv up to ALIAS (BAD_SHAPE, UNSUPPORTED_D,
 * BAD_SCALE, empty -> OK, NULL_PTR, MISALIGNED, ALIAS), then
 * ATTN_SCRATCH_TOO_SMALL when attn_fwd_splitkv_workspace_bytes() of the
 * call exceeds attn_noalloc_scratch_bytes() (no HIP call is made), then
 * ATTN_HIP (the lookup or the launch failed).  When one key range results
 * the scratch is not used.
 */
ATTN_API int attn_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                             int causal, float scale, int64_t num_splits, void *stream);

/* Size in bytes of attn_fwd_splitkv_noalloc's scratch array (per GPU). */
ATTN_API int64_t attn_noalloc_scratch_bytes(void);

/* Bytes of workspace attn_fwd_splitkv needs (0 for num_splits == 1);
 * -1 if the arguments are invalid (negative, d not 64/128, num_splits < 1,
 * or the size overflows). */
ATTN_API int64_t attn_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t d,
                                          int64_t num_splits);

/*
 * attn_bwd -- gradients of attn_fwd: dQ, dK and dV for an upstream gradient
 * dO, by recomputing the scores and probabilities tile by tile from the
 * forward pass's LSE instead of storing them (recomputation paragraph of
 * "FlashAttention evolution", letsgetai.github.io; "FlashAttention" concept
 * page, compassingai.com, section 3).  With P_ij = exp(scale q_i . k_j -
 * LSE_i) over the visible keys (the causal rule of attn_fwd) and
 * D_i = dO_i . O_i:
 *
 *   dV_j = sum_i P_ij dO_i
 *   dS_ij = P_ij (dO_i . v_j - D_i)
 *   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
 *
 * (bf16 out; fp32 arithmetic, P and dS rounded to bf16 as matrix-core
 * operands).  Results are deterministic: no atomics, the same bits for the
 * same inputs.
 *
 * q, k, v  the forward call's inputs: bf16, contiguous [B][H][N][d].
 * o, lse   the forward call's outputs for the same q, k, v, causal and scale
 *          (lse is required here): o bf16 [B][H][N][d], lse fp32 [B][H][N].
 * dout     dO, bf16 [B][H][N][d].
 * dq, dk, dv  bf16 [B][H][N][d], fully overwritten.
 * B, H, N, d, causal, scale, stream  as attn_fwd.
 * workspace, workspace_bytes  device scratch of at least
 *          attn_bwd_workspace_bytes(B, H, N, d) bytes (8 per row: the LSE in
 *          log2 units and D), 16-byte aligned, owned by the caller; contents
 *          on entry ignored, on return undefined; two calls in flight must
 *          not share one.
 * Ownership and asynchrony as attn_fwd (two kernels are enqueued).  Errors
 * are checked in the order of attn_fwd: BAD_SHAPE, UNSUPPORTED_D, BAD_SCALE,
 * (empty -> OK), NULL_PTR (any of the nine tensors), MISALIGNED (the bf16
 * tensors and the workspace 16 bytes, lse 4 bytes), ALIAS (dq, dk or dv
 * overlapping an input or each other; the inputs may alias one another),
 * BAD_WORKSPACE (NULL, misaligned, too small, or overlapping any tensor).
 */
ATTN_API int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dout, void *dq, void *dk, void *dv,
             int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
             void *workspace, int64_t workspace_bytes, void *stream);

/* Bytes of workspace attn_bwd needs (8 B H N); -1 if the arguments are
 * invalid (negative, d not 64/128, or the size overflows). */
ATTN_API int64_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * FP8 forward (head dim 128): block quantization with incoherent processing,
 * then attention on the FP8 operands -- the FP8 mode of FlashAttention-3
 * ("FlashAttention evolution", letsgetai.github.io, FlashAttention-3 section
 * and results; "FlashAttention 1-4 evolution cheat sheet", argus-lessons,
 * FlashAttention-3 section).  An approximation of attn_fwd, not an exact
 * result: inputs and P are rounded to FP8.
 *
 * Formats.  FP8 is OCP E4M3 (round to nearest even).  Rows are quantized in
 * blocks of 64 consecutive rows of one head; a block's scale is 2^E, E the
 * smallest integer with max|x| <= 448 * 2^E, stored as one E8M0 byte E + 127
 * per block: [B][H][Np / 64], Np = attn_fp8_padded_rows(N) = N rounded up
 * to 64.  Q and K are [B][H][Np][128] bytes, V is stored transposed as
 * [B][H][128][Np] with the keys of every 64-key tile permuted (key r at
 * position 32 ((r >> 2) & 1) + 16 (r >> 5) + 4 ((r >> 3) & 3) + (r & 3)),
 * which is the order the kernel's P V product consumes them in.  Rows
 * (keys) past N are zero.
 */
ATTN_API int64_t attn_fp8_padded_rows(int64_t N);

/*
 * attn_fp8_quantize -- bf16 x [B][H][N][128] (device, 16-byte aligned) to
 * FP8: out gets [B][H][Np][128] bytes (transpose == 0) or the permuted
 * [B][H][128][Np] V layout (transpose != 0); exps gets [B][H][Np / 64] E8M0
 * bytes.  sign_bits: NULL, or a HOST array of 4 words whose bit c (word
 * c / 32, bit c % 32) set makes column c's sign -1: then each row is first
 * rotated, x -> (x * s) H with H the 128 x 128 Sylvester Hadamard matrix
 * (+-1 entries, no 1/sqrt(128)), computed in fp32 by the fast transform with
 * strides 1, 2, ..., 64.  Q and K rotated with the same signs keep their
 * product times 128 (attn_fp8_quantize_q divides it out of Q).  This call
 * quantizes K and V for attn_fwd_fp8 (Q: attn_fp8_quantize_q).  Errors:
 * BAD_SHAPE, UNSUPPORTED_D (d != 128), BAD_ARGUMENT (signs with transpose),
 * (empty -> OK), NULL_PTR, MISALIGNED, ALIAS.  One kernel on `stream`.
 */
ATTN_API int attn_fp8_quantize(const void *x, int64_t B, int64_t H, int64_t N, int64_t d, int transpose,
                      const uint32_t *sign_bits, void *out, void *exps, void *stream);

/*
 * attn_fp8_quantize_q -- Q's quantization for attn_fwd_fp8: attn_fp8_quantize
 * with transpose == 0, except that after the rotation every value is
 * multiplied in fp32 by c = scale * log2(e) (one fp32 product), and by a
 * further 1/128 when sign_bits is given (the rotated Q K product carries the
 * Hadamard factor 128).  Q K^T of the quantized operands is then the logits
 * scale * q . k in log2 units, which attn_fwd_fp8 takes as they are.  scale
 * is the softmax scale of the original (unrotated) Q and K, e.g.
 * 1/sqrt(128); any finite value, zero and negative included.  Errors as
 * attn_fp8_quantize, and BAD_SCALE for a scale that is not finite.
 */
ATTN_API int attn_fp8_quantize_q(const void *x, int64_t B, int64_t H, int64_t N, int64_t d,
                        const uint32_t *sign_bits, float scale, void *out, void *exps, void *stream);

/*
 * attn_fwd_fp8 -- O (bf16 [B][H][N][128]) and LSE (fp32 [B][H][N] or NULL)
 * of softmax(scale * Q K^T) V from the FP8 operands: q8 and q_exps from
 * attn_fp8_quantize_q (which folds the softmax scale, log2(e) and the
 * rotation's factor into Q), k8 and vt8 (transposed) and their exponents
 * from attn_fp8_quantize, Q and K rotated with the same sign_bits or both
 * not rotated (incoherent processing).  Both products run on the FP8 matrix
 * cores with the block scales applied by the hardware; P is rounded to E4M3
 * for the P V product and O is divided by the fp32 sum of the unrounded P.
 * causal, stream as attn_fwd.  Errors as attn_fwd without BAD_SCALE
 * (d != 128 is UNSUPPORTED_D); one kernel on `stream`.
 */
ATTN_API int attn_fwd_fp8(const void *q8, const void *k8, const void *vt8, const void *q_exps,
                 const void *k_exps, const void *v_exps, void *o, float *lse,
                 int64_t B, int64_t H, int64_t N, int64_t d, int causal, void *stream);

/* Static, human-readable name of a status code ("ATTN_OK", ...). */
ATTN_API const char *attn_status_string(int status);

/* The hipError_t of the last call on this thread that returned ATTN_HIP
 * (0 if none has). */
ATTN_API int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_ATTN_H */
