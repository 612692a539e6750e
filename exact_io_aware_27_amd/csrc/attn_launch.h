// attn_launch.h -- internal interface between the validating C ABI
// (attn_api.hip) and the gfx950 kernels (attn_fwd_kernel.hip,
// attn_bwd_kernel.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Arguments of one validated call.  Sizes are already checked: d is 64 or
// 128, Nq * d and Nk * d are below 2^31, Nq <= Nk under the causal mask, and
// the workgroup count fits in an int.
struct AttnLaunch {
    const void *q, *k, *v;  // q: [BH][Nq][d]; k, v: [BH][Nk][d]
    void *o;                // [BH][Nq][d]
    float *lse;             // [BH][Nq] or null
    int64_t BH, Nq, Nk, d;
    bool causal;
    float scale;
    int64_t num_splits;  // key ranges; 1 = one pass straight into o and lse
    void *workspace;     // num_splits > 1: attn_splitkv_workspace_bytes() bytes
    hipStream_t stream;
};

// Keys per split range (a multiple of 128) and the number of non-empty
// ranges that num_splits asks for.
int64_t attn_split_keys(int64_t Nk, int64_t num_splits);
int64_t attn_splits_used(int64_t Nk, int64_t num_splits);

// Bytes of workspace a split call needs: fp32 O and LSE of every range.
int64_t attn_splitkv_workspace_bytes(int64_t BH, int64_t Nq, int64_t d, int64_t num_splits);

// An upper bound on the workgroups one call launches.
int64_t attn_workgroups(int64_t BH, int64_t Nq, int64_t Nk, int64_t num_splits);

// Enqueue the kernel(s); returns hipGetLastError() after the launches.
hipError_t attn_launch(const AttnLaunch &a);

// Key ranges of a call with at most kDecodeRows query rows per head:
// writes every range's normalised fp32 O and LSE into the split workspace
// (the layout of the forward kernel's split mode), for the merge kernel.
constexpr int64_t kDecodeRows = 4;
hipError_t attn_decode_ranges_launch(const AttnLaunch &a, int splits, int split_keys);

// Arguments of one validated backward call (attn_bwd).  d is 64 or 128,
// N * d is below 2^31 and the workgroup count fits in an int.
struct AttnBwdLaunch {
    const void *q, *k, *v, *o, *dout;  // [BH][N][d] bf16
    const float *lse;                  // [BH][N], natural log
    void *dq, *dk, *dv;                // [BH][N][d] bf16
    void *workspace;                   // attn_bwd_workspace_bytes() bytes
    int64_t BH, N, d;
    bool causal;
    float scale;
    hipStream_t stream;
};

// Workgroups of each backward kernel (an upper bound over masks).
int64_t attn_bwd_workgroups(int64_t BH, int64_t N);

// Enqueue the two backward kernels; returns hipGetLastError() after them.
hipError_t attn_bwd_launch(const AttnBwdLaunch &a);

// FP8 path (head dim 128).  Padded rows per head: N rounded up to 64.
int64_t attn_fp8_rows(int64_t N);

// One validated attn_fp8_quantize call.
struct AttnFp8Quantize {
    const void *x;               // [BH][N][128] bf16
    void *out, *exps;            // FP8 bytes and E8M0 block exponents
    const uint32_t *sign_bits;   // host, 4 words, or null (no rotation)
    bool transpose;              // V^T layout (no rotation)
    float mul;                   // fp32 multiplier after the rotation (1: none)
    int64_t BH, N;
    hipStream_t stream;
};
hipError_t attn_fp8_quantize_launch(const AttnFp8Quantize &q);

// One validated attn_fwd_fp8 call.
struct AttnFp8Launch {
    const void *q8, *k8, *vt8, *qe, *ke, *ve;
    void *o;
    float *lse;
    int64_t BH, N;
    bool causal;
    hipStream_t stream;
};
hipError_t attn_fp8_launch(const AttnFp8Launch &a);
