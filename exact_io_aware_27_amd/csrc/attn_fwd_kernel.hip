// attn_fwd_kernel.hip -- fused exact attention forward pass for gfx950.
//
// One workgroup owns one (batch*head, query tile) pair and walks the key/value
// tiles of that head in order (the FlashAttention-2 loop order and sequence
// parallelism: "FlashAttention 1-4 evolution cheat sheet", argus-lessons,
// FlashAttention-2 section).  Per key/value tile it forms the score tile on
// the matrix cores, updates the running row max m and running sum l, rescales
// the output accumulator by exp(m_old - m_new) and adds P V (the online
// softmax iteration of the "FlashAttention" concept page, compassingai.com,
// section 3, and the two-block merge equation of "FlashAttention evolution",
// letsgetai.github.io, core-mechanism section).  O is divided by l once, at
// the end.  Scores and probabilities live only in registers.
//
// gfx950 mapping
//   * 4 waves of 64 lanes, 32 query rows per wave, 128 per workgroup.
//   * Each wave computes the TRANSPOSED score tile S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator layout a lane holds
//     one column (here: one query) and 16 of the 32 rows (keys).  The row
//     max and row sum of a query are therefore 16 in-lane values plus one
//     exchange with the lane 32 apart (v_permlane32_swap), and the rescale
//     factor exp(m_old - m_new) is one scalar per lane.
//   * The probabilities leave the accumulator already in the register order
//     the next MFMA wants as its B operand, so O^T = V^T P^T needs no shuffle;
//     V is stored transposed in LDS so the A operand is two 8-byte reads.
//   * exp is v_exp_f32 (base 2): the scale is folded with log2(e) into one
//     multiplier, LSE is converted back with ln 2.
//   * K/V tiles of 64 keys are double-buffered in LDS with an XOR swizzle
//     that keeps the MFMA operand reads free of bank conflicts.
//   * Causal: tiles entirely above the diagonal are never loaded; the mask
//     is applied only in tiles that cross the diagonal or the sequence end.
//   * Workgroup order: heaviest causal query tiles first (longest-processing-
//     time order, "FlashAttention 1-4 evolution cheat sheet", FlashAttention-4
//     section), and the tiles of one head kept on one XCD so that its K/V
//     stream is shared through that XCD's L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn_gfx950 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kRowsPerWave * kWaves;  // query rows per workgroup
constexpr int kBc = 64;                     // keys per K/V tile
constexpr int kXcds = 8;                    // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr float kNegInf = -__builtin_inff();

template <int D>
struct Tile {
    static constexpr int kChunks = D / 8;            // 16-byte chunks per K row
    static constexpr int kKBytes = kBc * D * 2;      // K tile, row-major [key][d]
    static constexpr int kVBytes = kBc * D * 2;      // V tile, transposed [d][key]
    static constexpr int kStage = kKBytes + kVBytes; // one LDS buffer
    static constexpr int kQkSteps = D / 16;          // MFMA k-steps of Q K^T
    static constexpr int kOBlocks = D / 32;          // 32-row blocks of O^T
    static constexpr int kKPasses = kBc * kChunks / kThreads;
    static constexpr int kVThreads = (kBc / 4) * kChunks;  // threads staging V
};

// K tile in LDS: row r (a key) is D*2 bytes; its 16-byte chunk c lives at
// chunk position c ^ swz(r).  Any 8 aligned consecutive rows, and any 16,
// read at one logical chunk land on distinct bank groups.
template <int D>
__device__ __forceinline__ int k_offset(int r, int c)
{
    const int s = (D == 128) ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1));
    return r * (D * 2) + ((c ^ s) << 4);
}

// V^T tile in LDS: row dd (a head-dim index) is kBc*2 = 128 bytes = 16 units
// of 8 bytes (4 keys each); unit u lives at unit position u ^ swz(dd).
__device__ __forceinline__ int v_offset(int dd, int u)
{
    const int s = (dd & 15) ^ ((dd >> 4) & 1);
    return dd * (kBc * 2) + ((u ^ s) << 3);
}

// v_permlane32_swap_b32 a, b exchanges lanes 32..63 of a with lanes 0..31 of
// b.  Starting from a = b = x this leaves a = [x_lo, x_lo], b = [x_hi, x_hi],
// so op(a, b) combines lane l with lane l^32 in every lane.  Inline asm keeps
// the two results apart: the compiler builtin called with one value for both
// operands gets folded as if its two results were equal.
__device__ __forceinline__ void half_swap(float &a, float &b)
{
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ float wave_half_max(float x)
{
    // Lanes l and l^32 hold the two halves of one query's keys.
    float a = x, b = x;
    half_swap(a, b);
    return fmaxf(a, b);
}

__device__ __forceinline__ float wave_half_sum(float x)
{
    float a = x, b = x;
    half_swap(a, b);
    return a + b;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));  // RNE
}

// Logical workgroup order: XCD-major (consecutive logical indices share an
// XCD), then head-major, then query tiles from the last (heaviest under the
// causal mask) to the first.
__device__ __forceinline__ void tile_of(int wg, int n_wg, int nqt, int &bh, int &qt)
{
    const int xcd = wg % kXcds;
    const int slot = wg / kXcds;
    const int per = n_wg / kXcds;
    const int extra = n_wg % kXcds;
    const int lin = xcd * per + (xcd < extra ? xcd : extra) + slot;
    bh = lin / nqt;
    qt = nqt - 1 - lin % nqt;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    __bf16 *__restrict__ O, float *__restrict__ LSE, int N, int n_wg, int nqt, float c_log2)
{
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) char smem[2 * T::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n = lane & 31;     // this lane's query column in the 32x32 tiles
    const int half = lane >> 5;  // which half of the 32 keys / 16 k-values

    int bh, qt;
    tile_of(blockIdx.x, n_wg, nqt, bh, qt);
    const int q0 = qt * kBr;
    const size_t head = (size_t)bh * (size_t)N * D;
    const __bf16 *Qh = Q + head;
    const __bf16 *Kh = K + head;
    const __bf16 *Vh = V + head;

    const int qidx = q0 + wave * kRowsPerWave + n;
    const bool q_ok = qidx < N;

    // Q^T operand, resident for the whole key loop: k-step s holds
    // q[qidx][16 s + 8 half .. +7].
    bf16x8 qop[T::kQkSteps];
#pragma unroll
    for (int s = 0; s < T::kQkSteps; ++s) {
        if (q_ok)
            qop[s] = *reinterpret_cast<const bf16x8 *>(Qh + (size_t)qidx * D + 16 * s + 8 * half);
        else
            qop[s] = bf16x8{};
    }

    const int kv_end = CAUSAL ? min(N, q0 + kBr) : N;
    const int ntiles = (kv_end + kBc - 1) / kBc;

    // ---- global -> register staging of one K/V tile ----
    u32x4 kreg[T::kKPasses];
    u32x4 vreg[4];
    const int vc = tid % T::kChunks;  // V staging: 8 head-dim values ...
    const int vg = tid / T::kChunks;  // ... of 4 consecutive keys
    const bool v_stager = tid < T::kVThreads;

    auto load_tile = [&](int t) {
        const int kv0 = t * kBc;
#pragma unroll
        for (int p = 0; p < T::kKPasses; ++p) {
            const int idx = p * kThreads + tid;
            const int r = idx / T::kChunks, c = idx % T::kChunks;
            const int key = kv0 + r;
            kreg[p] = key < N ? *reinterpret_cast<const u32x4 *>(Kh + (size_t)key * D + 8 * c) : u32x4{};
        }
        if (v_stager) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kv0 + 4 * vg + i;
                // Rows past the end must be exact zeros: their P is 0, and 0 * NaN is NaN.
                vreg[i] = key < N ? *reinterpret_cast<const u32x4 *>(Vh + (size_t)key * D + 8 * vc)
                                  : u32x4{};
            }
        }
    };

    auto store_tile = [&](int buf) {
        char *ks = smem + buf * T::kStage;
        char *vs = ks + T::kKBytes;
#pragma unroll
        for (int p = 0; p < T::kKPasses; ++p) {
            const int idx = p * kThreads + tid;
            const int r = idx / T::kChunks, c = idx % T::kChunks;
            *reinterpret_cast<u32x4 *>(ks + k_offset<D>(r, c)) = kreg[p];
        }
        if (v_stager) {
            // Transpose the 4 keys x 8 head-dims block: head-dim j of keys
            // 4vg..4vg+3 becomes one 8-byte unit of V^T row 8vc + j.
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int w = j >> 1;
                uint32_t a0 = vreg[0][w], a1 = vreg[1][w], a2 = vreg[2][w], a3 = vreg[3][w];
                u32x2 out;
                if (j & 1) {
                    out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                    out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
                } else {
                    out[0] = (a0 & 0xffffu) | (a1 << 16);
                    out[1] = (a2 & 0xffffu) | (a3 << 16);
                }
                *reinterpret_cast<u32x2 *>(vs + v_offset(8 * vc + j, vg)) = out;
            }
        }
    };

    f32x16 oacc[T::kOBlocks];
#pragma unroll
    for (int b = 0; b < T::kOBlocks; ++b)
        oacc[b] = f32x16{};
    float m_run = kNegInf;  // running max, log2 units (scores times c_log2)
    float l_run = 0.f;      // running sum over this lane's half of the keys

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int kv0 = t * kBc;
        if (t + 1 < ntiles)
            load_tile(t + 1);  // global loads in flight during this tile's math

        const char *ks = smem + buf * T::kStage;
        const char *vs = ks + T::kKBytes;

        // S^T = K Q^T for two 32-key sub-blocks.
        f32x16 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            s[sb] = f32x16{};
            const int r = sb * 32 + n;
#pragma unroll
            for (int st = 0; st < T::kQkSteps; ++st) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ks + k_offset<D>(r, 2 * st + half));
                s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[st], s[sb], 0, 0, 0);
            }
        }

        // Scale into log2 units, mask, row max.  Register 4j+i of sub-block
        // sb holds key kv0 + 32 sb + 8 j + 4 half + i.
        const bool need_mask = (kv0 + kBc > N) || (CAUSAL && kv0 + kBc - 1 > q0);
        float mx = kNegInf;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[sb][r] * c_log2;
                if (need_mask) {
                    const int key = kv0 + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (key >= N || (CAUSAL && key > qidx))
                        x = kNegInf;
                }
                s[sb][r] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = wave_half_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // all-masked so far: no NaN
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float rowsum = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[sb][r] - m_use);
                s[sb][r] = p;
                rowsum += p;  // l sums fp32 p, before the bf16 rounding used by P V
            }
        }
        l_run = alpha * l_run + rowsum;
        m_run = m_new;
#pragma unroll
        for (int b = 0; b < T::kOBlocks; ++b)
            oacc[b] *= alpha;

        // O^T += V^T P^T: k-step ks2 of sub-block sb covers keys
        // 32 sb + 16 ks2 + {0..15}; position 8 half + 4 jj + i of both
        // operands is key 32 sb + 16 ks2 + 8 jj + 4 half + i.
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
                uint32_t pw[4];
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    pw[w] = pack_bf16x2(s[sb][8 * ks2 + 2 * w], s[sb][8 * ks2 + 2 * w + 1]);
                const u32x4 pv = {pw[0], pw[1], pw[2], pw[3]};
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pv);
                const int u0 = 8 * sb + 4 * ks2 + half;
#pragma unroll
                for (int b = 0; b < T::kOBlocks; ++b) {
                    const int dd = 32 * b + n;
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(vs + v_offset(dd, u0));
                    const u32x2 hi = *reinterpret_cast<const u32x2 *>(vs + v_offset(dd, u0 + 2));
                    const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pb,
                                                                      oacc[b], 0, 0, 0);
                }
            }
        }

        if (t + 1 < ntiles)
            store_tile(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: O = O / l, LSE = ln2 * (m + log2 l).
    const float l_tot = wave_half_sum(l_run);
    if (!q_ok)
        return;
    const float inv = 1.f / l_tot;
    __bf16 *orow = O + head + (size_t)qidx * D;
#pragma unroll
    for (int b = 0; b < T::kOBlocks; ++b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x2 w;
            w[0] = pack_bf16x2(oacc[b][4 * j + 0] * inv, oacc[b][4 * j + 1] * inv);
            w[1] = pack_bf16x2(oacc[b][4 * j + 2] * inv, oacc[b][4 * j + 3] * inv);
            *reinterpret_cast<u32x2 *>(orow + 32 * b + 8 * j + 4 * half) = w;
        }
    }
    if (LSE != nullptr && half == 0)
        LSE[(size_t)bh * N + qidx] = (m_run + __builtin_log2f(l_tot)) * 0.69314718055994530942f;
}

template <int D, bool CAUSAL>
static hipError_t launch(const AttnLaunch &a)
{
    const int nqt = (int)((a.N + kBr - 1) / kBr);
    const int n_wg = (int)(a.BH * nqt);
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL>), dim3(n_wg), dim3(kThreads), 0, a.stream,
                       (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v, (__bf16 *)a.o, a.lse,
                       (int)a.N, n_wg, nqt, a.scale * 1.44269504088896340736f);
    return hipGetLastError();
}

}  // namespace attn_gfx950

int64_t attn_workgroups(int64_t BH, int64_t N)
{
    return BH * ((N + attn_gfx950::kBr - 1) / attn_gfx950::kBr);
}

hipError_t attn_launch(const AttnLaunch &a)
{
    using namespace attn_gfx950;
    if (a.d == 128)
        return a.causal ? launch<128, true>(a) : launch<128, false>(a);
    return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}
