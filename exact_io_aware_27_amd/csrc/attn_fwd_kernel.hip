// attn_fwd_kernel.hip -- fused exact attention forward pass for gfx950.
//
// One workgroup owns one (batch*head, query tile) pair and walks the key/value
// tiles of that head in order (the FlashAttention-2 loop order and sequence
// parallelism: "FlashAttention 1-4 evolution cheat sheet", argus-lessons,
// FlashAttention-2 section).  Per key/value tile it forms the score tile on
// the matrix cores, keeps a running row max m and running sum l, rescales the
// output accumulator by exp(m_old - m_new) and adds P V (the online softmax
// iteration of the "FlashAttention" concept page, compassingai.com, section 3,
// and the two-block merge equation of "FlashAttention evolution",
// letsgetai.github.io, core-mechanism section).  O is divided by l once, at
// the end.  Scores and probabilities live only in registers.
//
// gfx950 mapping
//   * 4 waves of 64 lanes, 32 query rows per wave, 128 per workgroup, two
//     workgroups per CU.
//   * Each wave computes the TRANSPOSED score tile S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator layout a lane holds
//     one column (one query) and 16 of the 32 rows (keys), so a query's row
//     max and row sum are in-lane work plus one exchange with the lane 32
//     apart (v_permlane32_swap), and the rescale factor is one scalar per lane.
//   * The probabilities leave the accumulator in the register order the PV
//     MFMA wants for its B operand (O^T = V^T P^T), with no shuffle.
//   * K and V tiles of 64 keys go straight from global memory to LDS
//     (global_load_lds_dwordx4: no registers, no VALU), row-major with an XOR
//     swizzle of 16-byte chunks.  K feeds the QK^T MFMA with ds_read_b128;
//     V^T feeds the PV MFMA with ds_read_b64_tr_b16, the gfx950 transposing
//     LDS read (within 16 lanes it hands lane j the element j%4 of source
//     lanes j/4 + 4e), so V is never transposed in registers.
//   * Software pipeline inside each wave: while the VALU computes the softmax
//     of tile t, the matrix cores run Q K^T of tile t+1 and P V of tile t-1
//     (the GEMM/softmax overlap of "FlashAttention 1-4 evolution cheat
//     sheet", FlashAttention-3 section, done within one wave).  K is
//     prefetched two tiles ahead and V one tile ahead, double-buffered.
//   * exp is v_exp_f32 (base 2) with scale*log2(e) folded into one FMA.
//     The row max is exact at every 32-key block, so the largest probability
//     of a row is exactly 1 and rounds to bf16 without error; the O rescale
//     is skipped (a wave-uniform branch) when no row of the wave found a new
//     max, the common case once a few hundred keys have been seen.  (A
//     reference max that lags by up to 2^8, as in the conditional rescaling
//     of the FlashAttention-4 section, leaves the dominant probability
//     inexact in bf16 and breaks the 1e-2 bound on large-logit inputs.)
//   * Causal: tiles entirely above the diagonal are never loaded; the mask
//     is applied only in tiles that cross the diagonal or the sequence end.
//   * Workgroup order: heaviest causal query tiles first (longest-processing-
//     time order, FlashAttention-4 section of the cheat sheet), and the tiles
//     of one head kept on one XCD so that its K/V stream is shared through
//     that XCD's L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_launch.h"

namespace attn_gfx950 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

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
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;              // 16-byte chunks per row
    static constexpr int kBytes = kBc * kRowBytes;     // one K or V tile
    static constexpr int kQkSteps = D / 16;            // MFMA k-steps of Q K^T
    static constexpr int kOBlocks = D / 32;            // 32-row blocks of O^T
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows one wave-wide 16B load fills
    static constexpr int kLoadsPerWave = kBytes / 1024 / kWaves;
};

// Chunk c of row r sits at chunk position c ^ swz(r).
//  D = 128 (16 chunks): any 16 consecutive rows read at one chunk hit 16
//    distinct positions (ds_read_b128), and 4 aligned rows read as chunk
//    pairs {2u, 2u+1} hit 8 distinct positions (ds_read_b64_tr_b16).
//  D = 64 (8 chunks): any 8 aligned rows are distinct and 4 aligned rows
//    give distinct chunk pairs.
template <int D>
__device__ __forceinline__ int swz(int r)
{
    if constexpr (D == 128)
        return ((r & 7) << 1) | ((r >> 3) & 1);
    else
        return ((r & 3) << 1) | ((r >> 2) & 1);
}

template <int D>
__device__ __forceinline__ int tile_offset(int r, int c)
{
    return r * Tile<D>::kRowBytes + ((c ^ swz<D>(r)) << 4);
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

// Global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane L
// writes bytes [16 L, 16 L + 16) after the wave-uniform LDS address in M0.
// Issued through inline asm so the compiler does not treat it as a store that
// may alias every later LDS read (it would wait for it before each one); the
// kernel waits for these copies itself (s_waitcnt vmcnt before a barrier).
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr)
                 : "memory", "m0");
}

// One K or V tile (64 rows starting at key kv0) from global memory straight
// into LDS.  Wave w issues kLoadsPerWave wave-wide 16-byte loads; lane L of a
// load fills the L-th 16 bytes of its 1 KB slice, so the lane fetches the
// global chunk that the swizzle places there.  Rows past N are clamped to
// N-1: they are finite data whose probabilities are exactly 0.
template <int D>
__device__ __forceinline__ void load_tile(const __bf16 *src, int kv0, int N, uint32_t lds, int wave_u, int lane)
{
    using T = Tile<D>;
#pragma unroll
    for (int i = 0; i < T::kLoadsPerWave; ++i) {
        const int slice = wave_u * T::kLoadsPerWave + i;  // wave-uniform
        const int r = slice * T::kRowsPerLoad + lane / T::kChunks;
        const int pos = lane % T::kChunks;
        const int c = pos ^ swz<D>(r);
        const int key = min(kv0 + r, N - 1);
        lds_dma16(src + (size_t)key * D + c * 8, lds + slice * 1024);
    }
}

// S^T (32 keys x 32 queries) for the 32-key block at row rb of a K tile.
template <int D>
__device__ __forceinline__ f32x16 qk_block(const char *ks, int rb, const bf16x8 *qop, int n, int half)
{
    using T = Tile<D>;
    f32x16 s = {};
    const int r = rb + n;
#pragma unroll
    for (int st = 0; st < T::kQkSteps; ++st) {
        const bf16x8 a = *LDS_PTR(const bf16x8, ks + tile_offset<D>(r, 2 * st + half));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[st], s, 0, 0, 0);
    }
    return s;
}

// O^T += V^T P^T for the 32-key block at row rb of a V tile.  pb[ks] holds
// the bf16 probabilities of keys rb + 16 ks + {8 jj + 4 half + e} in operand
// position 8 half + 4 jj + e; the transposing reads hand the A operand the
// same key order (source lane i of a 16-lane group reads row i/4 of its 4-key
// group, head-dim columns 4 (i%4) .. +3).
template <int D>
__device__ __forceinline__ void pv_block(const char *vs, int rb, const bf16x8 *pb, f32x16 *oacc, int lane)
{
    using T = Tile<D>;
    const int g = lane >> 4;  // 16-lane group
    const int i = lane & 15;  // source lane within the group
    const int h = g >> 1;     // key half of the operand (lanes 32..63)
    const int dh = g & 1;     // which 16 of the block's 32 head-dim rows
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int b = 0; b < T::kOBlocks; ++b) {
            s16x4 part[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int r = rb + 16 * ks + 8 * jj + 4 * h + (i >> 2);
                const int dcol = 32 * b + 16 * dh + 4 * (i & 3);
                const int off = tile_offset<D>(r, dcol >> 3) + ((dcol & 4) << 1);
                part[jj] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vs + off));
            }
            const u32x2 lo = __builtin_bit_cast(u32x2, part[0]);
            const u32x2 hi = __builtin_bit_cast(u32x2, part[1]);
            const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
            oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pb[ks], oacc[b],
                                                              0, 0, 0);
        }
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    __bf16 *__restrict__ O, float *__restrict__ LSE, int N, int n_wg, int nqt, float c_log2)
{
    using T = Tile<D>;
    // K buffers 0, 1 then V buffers 0, 1.
    __shared__ __attribute__((aligned(1024))) char smem[4 * T::kBytes];
    const uint32_t smem_lds = (uint32_t)(uintptr_t)LDS_PTR(char, smem);
    auto kbuf = [&](int i) { return smem + i * T::kBytes; };
    auto vbuf = [&](int i) { return smem + (2 + i) * T::kBytes; };
    auto kbuf_lds = [&](int i) { return smem_lds + i * T::kBytes; };
    auto vbuf_lds = [&](int i) { return smem_lds + (2 + i) * T::kBytes; };

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int n = lane & 31;     // this lane's query column in the 32x32 tiles
    const int half = lane >> 5;  // which half of the 32 keys / 16 k-values

    int bh, qt;
    tile_of(blockIdx.x, n_wg, nqt, bh, qt);
    const int q0 = qt * kBr;
    const size_t head = (size_t)bh * (size_t)N * D;
    const __bf16 *Kh = K + head;
    const __bf16 *Vh = V + head;

    const int qw0 = q0 + wave * kRowsPerWave;  // first query of this wave
    const int qidx = qw0 + n;
    const bool q_ok = qidx < N;

    const int kv_end = CAUSAL ? min(N, q0 + kBr) : N;
    const int ntiles = (kv_end + kBc - 1) / kBc;
    const int nblocks = 2 * ntiles;  // 32-key pipeline steps

    // Prologue: K tiles 0 and 1 and V tile 0 in flight while Q is read.
    load_tile<D>(Kh, 0, N, kbuf_lds(0), wave_u, lane);
    if (ntiles > 1)
        load_tile<D>(Kh, kBc, N, kbuf_lds(1), wave_u, lane);
    load_tile<D>(Vh, 0, N, vbuf_lds(0), wave_u, lane);

    // Q^T operand, resident for the whole key loop: k-step s holds
    // q[qidx][16 s + 8 half .. +7] (zeros past N).
    bf16x8 qop[T::kQkSteps];
    {
        const __bf16 *qrow = Q + head + (size_t)min(qidx, N - 1) * D + 8 * half;
#pragma unroll
        for (int s = 0; s < T::kQkSteps; ++s) {
            qop[s] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * s);
            if (!q_ok)
                qop[s] = bf16x8{};
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x16 sc = qk_block<D>(kbuf(0), 0, qop, n, half);  // scores of block 0
    f32x16 oacc[T::kOBlocks];
#pragma unroll
    for (int b = 0; b < T::kOBlocks; ++b)
        oacc[b] = f32x16{};
    float m_ref = kNegInf;  // reference max, log2 units (scores times c_log2)
    float l_run = 0.f;      // running sum over this lane's half of the keys
    bf16x8 pb_prev[2] = {bf16x8{}, bf16x8{}};  // P of the previous block (none yet: zeros)

    // One 32-key pipeline step, straight-line code so that the softmax of
    // block k (VALU) interleaves with the scores of block k+1 and P V of block
    // k-1 (matrix cores).  At the ends the block indices are clamped: the
    // first step multiplies V block 0 by P = 0, the last recomputes scores it
    // discards.  MASKED steps apply the causal / sequence-end mask and also
    // serve non-positive scales.
    auto step = [&](int k, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int kq = min(k + 1, nblocks - 1);
        const int kp = max(k - 1, 0);
        const char *kq_buf = kbuf((kq >> 1) & 1);
        const int kq_row = 32 * (kq & 1);

        // K operands of block k+1, read early so their latency hides under the softmax.
        bf16x8 kop[T::kQkSteps];
#pragma unroll
        for (int st = 0; st < T::kQkSteps; ++st)
            kop[st] = *LDS_PTR(const bf16x8, kq_buf + tile_offset<D>(kq_row + n, 2 * st + half));

        // Register 4j+e holds key 32 k + 8 j + 4 half + e.
        float mx;
        if constexpr (!MASKED) {
            float r0 = sc[0];
#pragma unroll
            for (int r = 1; r < 16; ++r)
                r0 = fmaxf(r0, sc[r]);
            mx = r0 * c_log2;
        } else {
            mx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = sc[r] * c_log2;
                const int key = 32 * k + 8 * (r >> 2) + 4 * half + (r & 3);
                x = (key >= N || (CAUSAL && key > qidx)) ? kNegInf : x;
                sc[r] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = wave_half_max(mx);

        // Exact running max; O needs rescaling only if some row of the wave
        // found a new max in this block (always so on the first block).
        const float m_new = fmaxf(m_ref, mx);
        const bool rescale = __builtin_amdgcn_ballot_w64(m_new > m_ref) != 0;  // wave-uniform
        const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;  // all masked so far: p = 0, no NaN
        // Unmasked blocks hold raw scores (p = exp2(s c - m)); masked ones hold s c already.
        const float cmul = MASKED ? 1.f : c_log2;

        float rowsum = 0.f;
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], cmul, -m_use));
            rowsum += p[r];  // l sums fp32 p, before the bf16 rounding used by P V
        }
        bf16x8 pb[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4 w = {pack_bf16x2(p[8 * ks + 0], p[8 * ks + 1]), pack_bf16x2(p[8 * ks + 2], p[8 * ks + 3]),
                             pack_bf16x2(p[8 * ks + 4], p[8 * ks + 5]), pack_bf16x2(p[8 * ks + 6], p[8 * ks + 7])};
            pb[ks] = __builtin_bit_cast(bf16x8, w);
        }

        f32x16 sn = {};
#pragma unroll
        for (int st = 0; st < T::kQkSteps; ++st)
            sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[st], qop[st], sn, 0, 0, 0);
        pv_block<D>(vbuf((kp >> 1) & 1), 32 * (kp & 1), pb_prev, oacc, lane);
        sc = sn;

        l_run = alpha * l_run + rowsum;
        if (rescale) {  // after P V of block k-1, which was relative to the old reference
#pragma unroll
            for (int b = 0; b < T::kOBlocks; ++b)
                oacc[b] *= alpha;
        }
        pb_prev[0] = pb[0];
        pb_prev[1] = pb[1];
    };

    // One 64-key tile = two steps.  The even step makes the last reads of K
    // tile t and V tile t-1; after the barrier those buffers are refilled
    // with K tile t+2 and V tile t+1, which land before the next barrier.
    auto tile = [&](int t, auto masked_tag) {
        step(2 * t, masked_tag);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 2 < ntiles)
            load_tile<D>(Kh, (t + 2) * kBc, N, kbuf_lds(t & 1), wave_u, lane);
        if (t + 1 < ntiles)
            load_tile<D>(Vh, (t + 1) * kBc, N, vbuf_lds((t + 1) & 1), wave_u, lane);
        step(2 * t + 1, masked_tag);
    };

    // Tiles [0, t_free) need no mask: below the causal diagonal of every
    // query of the workgroup and wholly inside the sequence.
    int t_free = N / kBc;
    if (CAUSAL)
        t_free = min(t_free, (q0 + 1) / kBc);
    if (!(c_log2 > 0.f))
        t_free = 0;
    t_free = min(t_free, ntiles);
    for (int t = 0; t < t_free; ++t)
        tile(t, std::false_type{});
    for (int t = t_free; t < ntiles; ++t)
        tile(t, std::true_type{});
    pv_block<D>(vbuf((ntiles - 1) & 1), 32, pb_prev, oacc, lane);

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
        LSE[(size_t)bh * N + qidx] = (m_ref + __builtin_log2f(l_tot)) * 0.69314718055994530942f;
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
