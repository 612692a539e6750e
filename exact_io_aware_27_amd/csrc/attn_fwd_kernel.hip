// attn_fwd_kernel.hip -- fused exact attention forward pass for gfx950.
//
// A workgroup owns a query tile of one batch*head (two, in turn, under the
// causal mask) and walks the key/value tiles of that head in order (the FlashAttention-2 loop order and sequence
// parallelism: "FlashAttention 1-4 evolution cheat sheet", argus-lessons,
// FlashAttention-2 section).  Per key/value block it forms the score tile on
// the matrix cores, keeps a running row max m and running sum l, rescales the
// output accumulator by exp(m_old - m_new) and adds P V (the online softmax
// iteration of the "FlashAttention" concept page, compassingai.com, section 3,
// and the two-block merge equation of "FlashAttention evolution",
// letsgetai.github.io, core-mechanism section).  O is divided by l once, at
// the end.  Scores and probabilities live only in registers.
//
// gfx950 mapping
//   * 32 query rows per 64-lane wave.  d = 128: 8 waves (256 queries) per
//     workgroup, one workgroup per CU; key ranges of a few query rows
//     (decoding) at d = 128: 4 waves (128 queries), two workgroups per CU;
//     either way two waves share each SIMD.  d = 64: 4 waves, three
//     workgroups per CU (three waves per SIMD).
//   * Each wave computes the TRANSPOSED score tile S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator layout a lane holds
//     one column (one query) and 16 of the 32 rows (keys), so a query's row
//     max and row sum are in-lane work plus one exchange with the lane 32
//     apart (v_permlane32_swap), and the rescale factor is one scalar per lane.
//   * The probabilities leave the accumulator in the register order the PV
//     MFMA wants for its B operand (O^T = V^T P^T), with no shuffle.
//   * K and V tiles of 64 keys go straight from global memory to LDS
//     (buffer_load_dwordx4 ... lds: no registers, no VALU; a fixed per-lane
//     offset plus a per-tile SGPR offset, range-checked against the head so
//     rows past N read as zeros), row-major with an XOR swizzle of 16-byte
//     chunks.  The four LDS buffers are separate arrays, so the compiler can
//     see that a copy into one buffer never aliases reads of another and
//     schedules the copies among the MFMAs of a step without waiting on
//     them.  K feeds the QK^T MFMA with ds_read_b128; V^T feeds the PV MFMA
//     with ds_read_b64_tr_b16, the gfx950 transposing LDS read (within 16
//     lanes it hands lane j the element j%4 of source lanes j/4 + 4e), so V
//     is never transposed in registers.
//   * Software pipeline inside each wave, in 32-key steps: while the VALU
//     computes the softmax of block k, the matrix cores run Q K^T of block
//     k+1 and P V of block k-1 (the GEMM/softmax overlap of "FlashAttention
//     1-4 evolution cheat sheet", FlashAttention-3 section, done within one
//     wave), with an explicit interleave of MFMAs, VALU work and operand
//     reads.  K is prefetched two 64-key tiles ahead and V one tile ahead,
//     double-buffered, one barrier per tile.
//   * exp is v_exp_f32 (base 2) with scale*log2(e) folded into one FMA.
//     Probabilities are taken against a reference max that may lag the
//     exact running max by up to 16 (log2 units), the conditional rescaling
//     of the FlashAttention-4 section of the cheat sheet: the exps of a block
//     never wait for its own max.  Two guards keep p bounded, chosen per
//     instance by measurement.  The causal instances and d = 64 check each
//     block's own sums after the exps (3 instructions per step); the rare,
//     wave-uniform branch moves the reference to the row's exact running
//     max, rescales l, lb and O, and takes the block again from its scores.
//     The non-causal d = 128 instances compute the row max of the NEXT
//     block from its fresh scores (during the P V MFMAs); a row that would
//     pass the slack moves the reference to its exact max, and the rare
//     branch rescales the sums at once and O after the next P V.  With a lagging
//     reference the largest p is not 1 and its bf16 rounding is not exact,
//     so O is divided by the sum of the bf16-rounded probabilities that
//     built it (v_dot2c_f32_bf16 against ones), which keeps a one-hot row
//     exact; the LSE uses the fp32 sum.
//   * Causal: tiles entirely above the diagonal are never loaded; the mask
//     is applied only in tiles that cross the diagonal or the sequence end.
//   * Causal load balance: a workgroup runs two query tiles of one head in
//     turn, tile nqt-1-j and then tile j, so every workgroup walks nearly the
//     same number of key tiles and the launch ends without a tail of heavy
//     diagonal-far tiles (the balancing concern of the FlashAttention-4
//     section of the cheat sheet, met here by pairing instead of ordering).
//     Workgroups of one head stay on one XCD so that its K/V stream is shared
//     through that XCD's L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"
#include "exp2_poly.h"

// The FlashAttention-4 split of the softmax exponentials between the hardware
// exponential and a polynomial on the FMA units (cheat sheet, FlashAttention-4
// section), as a build option for measurement: with ATTN_EXP2_POLY_EVERY = n
// > 0, one exponential in every n of a block goes to exp2_poly.  The default
// build (0) keeps every exponential on v_exp_f32: on gfx950 both run on the
// same VALU, and the polynomial's 8 instructions cost more issue cycles than
// v_exp_f32 (bench.py --micro; the A/B with this option measured every split
// slower).
#ifndef ATTN_EXP2_POLY_EVERY
#define ATTN_EXP2_POLY_EVERY 0
#endif

namespace attn_gfx950 {

constexpr int kRowsPerWave = 32;
constexpr int kBrMin = 128;  // fewest query rows per workgroup (d = 64)
constexpr int kBc = 64;      // keys per K/V tile (two 32-key blocks)
// A block's probabilities are taken against a reference max that may lag
// the true running max by up to kRefSlack (log2 units): p <= 2^16.  Under the
// next-block guard a row whose next block would exceed that moves the
// reference to its exact max.
[[maybe_unused]] constexpr float kRefSlack = 16.f;
// Under the sum check a lane's 16 probabilities of one block may add up to
// at most 2^16 against the reference.
[[maybe_unused]] constexpr float kSumLimit = 65536.f;

// Workgroup shape per head dim.  d = 128: 8 waves (256 queries), one
// workgroup per CU, two waves per SIMD from the same workgroup: each K/V
// tile copied into LDS serves twice the queries, which halves the L2->LDS
// copy traffic per flop (the copies cost shader clock under the chip's power
// limit).  d = 64: 4 waves (128 queries), two workgroups per CU, so that the
// smaller d = 64 problems still fill the chip.  Split-key decoding at
// d = 128 (few query rows, so most waves of a workgroup only copy) takes
// 4 waves as well: two workgroups per CU then put two computing waves on
// every CU instead of one.
template <int D, int W = (D == 128 ? 8 : 4)>
struct Tile {
    static constexpr int kWaves = W;
    static constexpr int kThreads = kWave * kWaves;
    static constexpr int kBr = kRowsPerWave * kWaves;  // query rows per workgroup
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
    static constexpr int kBytes = kBc * kRowBytes;         // one K or V tile
    static constexpr int kQkSteps = D / 16;                // MFMA k-steps of Q K^T
    static constexpr int kOBlocks = D / 32;                // 32-row blocks of O^T
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows one wave-wide 16-byte load fills
    static constexpr int kLoadsPerWave = kBytes / 1024 / kWaves;
};

// LDS tiles are row-major (one key per row, D*2 bytes) with 16-byte chunk c
// of row r stored at chunk position c ^ swz(r).
//  K tiles (read by ds_read_b128, lanes 0..15 on 16 consecutive rows at one
//  chunk): D = 128 uses a 4-bit swizzle, distinct over any 16 consecutive
//  rows; D = 64 (8 chunks, two rows per 256 bytes) uses one distinct over
//  any aligned 8 rows and over (row parity, position) for 16 rows.
//  V tiles (read by ds_read_b64_tr_b16; the LDS serves 32 lanes per cycle:
//  4 aligned rows x the 4 chunks of one 32-column head-dim block): D = 128
//  (one row per 256 bytes) XORs (r & 3) into chunk bits 2..3, so the 4 rows
//  land on 4 distinct 64-byte bank blocks; D = 64 (two rows per 256 bytes)
//  needs rows r and r+2 apart, which bit 2 = (r >> 1) & 1 gives.
template <int D>
__device__ __forceinline__ int swz_k(int r)
{
    if constexpr (D == 128)
        return ((r & 7) << 1) | ((r >> 3) & 1);
    else
        return (r & 7) ^ ((r >> 3) & 1);
}

template <int D>
__device__ __forceinline__ int swz_v(int r)
{
    if constexpr (D == 128)
        return (r & 3) << 2;
    else
        return ((r & 3) << 1) | ((r >> 2) & 1);
}

template <int D>
__device__ __forceinline__ int k_offset(int r, int c)
{
    return r * Tile<D>::kRowBytes + ((c ^ swz_k<D>(r)) << 4);
}

template <int D>
__device__ __forceinline__ int v_offset(int r, int c)
{
    return r * Tile<D>::kRowBytes + ((c ^ swz_v<D>(r)) << 4);
}

// Kernel arguments.  Q, O, LSE: [BH][Nq](×d); K, V: [BH][Nk][d].  Under the
// causal mask query i sees key j iff j <= i + (Nk - Nq) (the queries are the
// last Nq positions of the sequence).  The key range [0, Nk) is cut into
// n_splits ranges of split_keys keys (a multiple of two 64-key tiles); with
// SPLIT each workgroup writes its range's normalised fp32 O and its LSE to
// Opart [n_splits][BH][Nq][d] and LSEpart [n_splits][BH][Nq] for the merge
// kernel, else bf16 O and fp32 LSE (LSE may be null) directly.
struct KArgs {
    const __bf16 *Q, *K, *V;
    __bf16 *O;
    float *LSE;
    float *Opart, *LSEpart;
    int BH, Nq, Nk, n_wg, nqt, n_splits, split_keys;
    int lpt;  // causal, one key range: single query tiles, longest first
    float c_log2;
};

// Waves per SIMD, stated as the register budget.  d = 128: two (one 8-wave
// workgroup per CU, 256 VGPRs each); without the statement the scheduler
// keeps a step in source order whenever the interleaved MFMA/softmax order
// would cross the three-wave register threshold (168 VGPRs), which costs up
// to 8%.  d = 64: three (three 4-wave workgroups per CU, 168 VGPRs, no VGPR
// spill): the short d = 64 launches spend much of a workgroup's life in its
// prologue, and a third resident workgroup hides more of it (same-box A/B,
// bitwise-equal output: +3-5% on every d = 64 shape measured, B=8 H=12
// N=1024 causal 457 -> 475 TFLOP/s).
template <int D>
constexpr int waves_per_simd()
{
    return D == 64 ? 3 : 2;
}

template <int D, bool CAUSAL, bool SPLIT, int W>
__global__ __launch_bounds__((Tile<D, W>::kThreads)) __attribute__((
    amdgpu_waves_per_eu(waves_per_simd<D>(), waves_per_simd<D>()))) void attn_fwd_kernel(
    const KArgs a)
{
    // The body is device code only (gfx950 buffer resources and LDS builtins);
    // the host pass needs just the declaration to emit the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    using T = Tile<D, W>;
    // The lagging reference's guard.  The check of each block's own sums
    // costs 3 instructions per step against the next block's row max (about
    // 11).  Same-box A/B, outputs bitwise equal: the long causal workload ran
    // 1099 -> 1150 TFLOP/s with the sum check (and 4 VALU per MFMA group,
    // below); the non-causal large-logit one 1124 -> 1097, as its compiled
    // step lost the MFMA interleave, so the non-causal d = 128 instances keep
    // the row max.  d = 64 is VALU-bound and has always used the sum check.
    constexpr bool kSumCheck = D == 64 || CAUSAL;
    // VALU instructions placed after each MFMA of a step: 16 x 4 covers the
    // sum-check step's softmax at d = 128 (about 71 instructions); 5 suits
    // the longer row-max step and d = 64.
    constexpr int kValuPerMfma = (D == 128 && kSumCheck) ? 4 : 5;
    // LDS: K buffers 0, 1 and V buffers 0, 1, each one 64-key tile, as four
    // separate arrays (see the header comment).
    __shared__ __attribute__((aligned(1024))) char sk0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char sk1[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char sv0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char sv1[T::kBytes];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int n = lane & 31;     // this lane's query column in the 32x32 tiles
    const int half = lane >> 5;  // which half of the 32 keys / 16 k-values

    const int Nq = a.Nq, Nk = a.Nk, nqt = a.nqt;
    const float c_log2 = a.c_log2;
    const int delta = Nk - Nq;  // causal offset: query i sees keys <= i + delta

    // Causal: unit j of a head is the pair of query tiles (nqt-1-j, j), the
    // heavy one first, so that every workgroup does nearly the same work (the
    // middle tile of an odd count is alone); non-causal: one tile per unit.
    // Work items are ordered (head, split, unit), so that all the work on one
    // head's keys stays on one XCD.
    //
    // A causal grid too small to fill the chip twice over with pairs (or a
    // few query tiles per head) runs single tiles instead, longest first
    // within each XCD: XCD x owns heads [x B H / 8, (x + 1) B H / 8), and its
    // workgroups walk them tile by tile from the heaviest (the host chooses
    // this only when 8 divides B H).  Uneven work then fills the slots the
    // pairs would have left idle.  The XCD's dispatch positions are dealt to
    // its CUs in rounds, so the rounds alternate direction (snake_slot): the
    // CU that takes the heaviest tile of one round takes the lightest of the
    // next, which evens out the work each CU holds (gpt2_small +3.4%,
    // bitwise-equal output).
    const bool lpt = CAUSAL && !SPLIT && a.lpt;
    const int n_units = (CAUSAL && !lpt) ? (nqt + 1) / 2 : nqt;
    int bh, rem;
    if (lpt) {
        const int hpx = a.BH / kXcds, xcd = blockIdx.x % kXcds;
        const int slot = snake_slot(blockIdx.x / kXcds, hpx * nqt);
        bh = xcd * hpx + slot % hpx;
        rem = (nqt - 1) - slot / hpx;
    } else {
        unit_of(blockIdx.x, a.n_wg, n_units * a.n_splits, bh, rem);
    }
    const int split = rem / n_units, unit = rem % n_units;
    const int kv_lo = split * a.split_keys;
    const int kv_hi = min(Nk, kv_lo + a.split_keys);
    const int npass = (CAUSAL && !lpt && nqt - 1 - unit != unit) ? 2 : 1;
    for (int pass = 0; pass < npass; ++pass) {
        const int qt = (CAUSAL && !lpt) ? (pass == 0 ? nqt - 1 - unit : unit) : unit;
        if (pass > 0)
            __syncthreads();  // every wave is done with the previous tile's LDS
        const int q0 = qt * T::kBr;
        const size_t qhead = (size_t)bh * (size_t)Nq * D;
        const size_t kvhead = (size_t)bh * (size_t)Nk * D;
        const __bf16 *Kh = a.K + kvhead;
        const __bf16 *Vh = a.V + kvhead;

        const int qw0 = q0 + wave * kRowsPerWave;  // first query of this wave
        const int qidx = qw0 + n;
        const bool q_ok = qidx < Nq;

        // This tile's keys in this split: [kv_lo, kv_end), in 64-key tiles
        // [t_lo, t_end); t_lo is even (split_keys is a multiple of 128).
        const int kv_end = CAUSAL ? min(kv_hi, q0 + T::kBr + delta) : kv_hi;
        const int t_lo = kv_lo / kBc;
        const int t_end = (kv_end + kBc - 1) / kBc;
        // Copies go through buffer resources over this head's keys [0, kv_end):
        // rows at or past kv_end (invisible to every query of the tile) are out
        // of range and read as zeros with no memory access, so the prefetches
        // past the end of the range cost nothing.
        // (N d < 2^31 keeps byte counts below 2^32: unsigned arithmetic.)
        const uint32_t head_bytes = (uint32_t)kv_end * (uint32_t)T::kRowBytes;

        // Result of rows that see no key of this range: LSE = -inf, O = 0.
        if (t_end <= t_lo) {
            if constexpr (SPLIT) {
                if (q_ok) {
                    float *op = a.Opart + (((size_t)split * a.BH + bh) * Nq + qidx) * D;
#pragma unroll
                    for (int b = 0; b < T::kOBlocks; ++b)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            *reinterpret_cast<f32x4 *>(op + 32 * b + 8 * j + 4 * half) = f32x4{};
                    if (half == 0)
                        a.LSEpart[((size_t)split * a.BH + bh) * Nq + qidx] = kNegInf;
                }
            }
            continue;
        }

        // ---- per-lane offsets, fixed for the whole loop ----
        // DMA: slice i of this wave is LDS bytes [1024 s, 1024 s + 1024) of a tile
        // (s = wave * kLoadsPerWave + i); the lane fetches row r, chunk c.
        uint32_t kdma[T::kLoadsPerWave], vdma[T::kLoadsPerWave];
#pragma unroll
        for (int i = 0; i < T::kLoadsPerWave; ++i) {
            const int slice = wave * T::kLoadsPerWave + i;
            const int r = slice * T::kRowsPerLoad + lane / T::kChunks;
            const int pos = lane % T::kChunks;
            kdma[i] = r * T::kRowBytes + ((pos ^ swz_k<D>(r)) << 4);
            vdma[i] = r * T::kRowBytes + ((pos ^ swz_v<D>(r)) << 4);
        }
        // K operand of S^T = K Q^T: row n of a 32-key block, chunk 2 st + half.
        uint32_t koff[T::kQkSteps];
#pragma unroll
        for (int st = 0; st < T::kQkSteps; ++st)
            koff[st] = k_offset<D>(n, 2 * st + half);
        // V^T operand through ds_read_b64_tr_b16: source lane i of 16-lane group
        // g reads key row 8 jj + 4 (g / 2) + i / 4 of a 16-key step, head-dim
        // columns 32 b + 16 (g % 2) + 4 (i % 4) .. +3.
        uint32_t voff[T::kOBlocks][2];
        {
            const int g = lane >> 4, i = lane & 15;
#pragma unroll
            for (int b = 0; b < T::kOBlocks; ++b)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int r = 8 * jj + 4 * (g >> 1) + (i >> 2);
                    const int dcol = 32 * b + 16 * (g & 1) + 4 * (i & 3);
                    voff[b][jj] = v_offset<D>(r, dcol >> 3) + ((dcol & 4) << 1);
                }
        }
        auto vread = [&](const char *buf, int byte, int b, int jj) __attribute__((always_inline)) {  // 4 keys x 1 head-dim column, transposed
            return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                LDS_PTR(s16x4, buf + byte + voff[b][jj]));
        };

        // One K or V tile (64 keys from kv0) into an LDS buffer: this wave's
        // kLoadsPerWave 1 KB slices, each one buffer_load_dwordx4 ... lds.  Rows
        // past kv_end, and whole tiles past it, read as zeros (no memory access),
        // so the copy needs no branch.
        auto load_tile = [&](const __bf16 *src, int kv0, char *buf, const uint32_t *dma) __attribute__((always_inline)) {
            const __amdgpu_buffer_rsrc_t rsrc =
                __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, (int)head_bytes, kBufferFlags);
#pragma unroll
            for (int i = 0; i < T::kLoadsPerWave; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, LDS_PTR(void, buf + (wave_u * T::kLoadsPerWave + i) * 1024), 16, dma[i],
                    (int)((uint32_t)kv0 * (uint32_t)T::kRowBytes), 0, 0);
        };

        // Prologue: K tiles t_lo and t_lo+1 and V tile t_lo in flight while Q is
        // read; V buffer 1 is zeroed for the first step's (empty) P V.
        load_tile(Kh, kv_lo, sk0, kdma);
        load_tile(Kh, kv_lo + kBc, sk1, kdma);
        load_tile(Vh, kv_lo, sv0, vdma);
#pragma unroll
        for (int i = 0; i < T::kBytes / (16 * T::kThreads); ++i)
            *LDS_PTR(u32x4, sv1 + 16 * (tid + i * T::kThreads)) = u32x4{};

        // Q^T operand, resident for the whole key loop: k-step s holds
        // q[qidx][16 s + 8 half .. +7] (zeros past Nq).
        bf16x8 qop[T::kQkSteps];
        {
            const __bf16 *qrow = a.Q + qhead + (size_t)min(qidx, Nq - 1) * D + 8 * half;
#pragma unroll
            for (int s = 0; s < T::kQkSteps; ++s) {
                qop[s] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * s);
                if (!q_ok)
                    qop[s] = bf16x8{};
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        f32x16 sc = {};  // scores of the block being turned into probabilities
#pragma unroll
        for (int st = 0; st < T::kQkSteps; ++st)
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*LDS_PTR(const bf16x8, sk0 + koff[st]), qop[st], sc, 0, 0, 0);
        f32x16 oacc[T::kOBlocks];
#pragma unroll
        for (int b = 0; b < T::kOBlocks; ++b)
            oacc[b] = f32x16{};
        // Key r of block kb (register r of the score tile) is visible to this
        // lane's query: inside this key range and, causal, not after the query.
        auto visible = [&](int kb, int r) __attribute__((always_inline)) {
            const int key = 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
            return !(key >= kv_hi || (CAUSAL && key > qidx + delta));
        };
        // Reference max m_ref of this lane's row (log2 units, scores times
        // c_log2), the value subtracted before exp2 (m_ref, or 0 while nothing
        // is visible) and the largest score the reference still serves.
        float m_ref, m_sub, m_thr;
        auto set_ref = [&](float m) __attribute__((always_inline)) {
            m_ref = m;
            m_sub = (m == kNegInf) ? 0.f : m;
            m_thr = m + kRefSlack;
        };
        {  // the range's first block sets the first reference: its exact row max
            // (keys counted from kv_lo: key kv_lo + kr is visible iff kr < kv_hi - kv_lo
            // and, causal, kr <= qidx + delta - kv_lo)
            const int lim_hi = kv_hi - kv_lo, lim_q = CAUSAL ? qidx + delta - kv_lo : 0x7fffffff;
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kr = 8 * (r >> 2) + 4 * half + (r & 3);
                mx = fmaxf(mx, (kr < lim_hi && kr <= lim_q) ? sc[r] * c_log2 : kNegInf);
            }
            set_ref(wave_half_max(mx));
        }
        float l_run = 0.f;       // sum of fp32 p over this lane's half of the keys
        float lb_run = 0.f;      // sum of the bf16-rounded p, same keys
        bool pending = false;    // O still to be rescaled by alpha_pend (wave-uniform)
        float alpha_pend = 1.f;
        bf16x8 pb_prev[2] = {bf16x8{}, bf16x8{}};  // P of the previous block (none yet: zeros)
        const bf16x2 kOnes = __builtin_bit_cast(bf16x2, 0x3f803f80u);  // bf16 {1, 1}

        // O^T += V^T P^T over the 32 keys of one block (two 16-key k-steps);
        // the block's first V row is at byte vp of V buffer vbuf.
        auto pv = [&](const char *vbuf, int vp, const bf16x8 *pbk) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int b = 0; b < T::kOBlocks; ++b) {
                    const int vb = vp + ks * 16 * T::kRowBytes;
                    const u32x2 lo = __builtin_bit_cast(u32x2, vread(vbuf, vb, b, 0));
                    const u32x2 hi = __builtin_bit_cast(u32x2, vread(vbuf, vb, b, 1));
                    const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pbk[ks], oacc[b],
                                                                      0, 0, 0);
                }
            }
        };

        // The probabilities of block k (scores s, reference m_sub): P as bf16 in
        // the B-operand order of the P V MFMA, the sum rs of the fp32 p and the
        // sum rb of the bf16-rounded p over this lane's 16 keys.
        // Register 4j+e holds key 32 k + 8 j + 4 half + e.
        auto block_softmax = [&](const f32x16 &s, float msub, int k, auto masked_tag, bf16x8 *pbo, float &rs,
                                 float &rb) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float x = __builtin_fmaf(s[r], c_log2, -msub);
                if (ATTN_EXP2_POLY_EVERY > 0 && r % (ATTN_EXP2_POLY_EVERY > 0 ? ATTN_EXP2_POLY_EVERY : 1) == ATTN_EXP2_POLY_EVERY - 1)
                    p[r] = exp2_poly(x);
                else
                    p[r] = __builtin_amdgcn_exp2f(x);
                if constexpr (MASKED)
                    p[r] = visible(k, r) ? p[r] : 0.f;
            }
            float rs0 = p[0], rs1 = p[1];
#pragma unroll
            for (int r = 2; r < 16; r += 2) {
                rs0 += p[r];
                rs1 += p[r + 1];
            }
            // The bf16 pairs are summed from the scalar words: summing from the
            // elements of the packed vector (w[e] in a loop) gets all four dot
            // products fed the first element by the compiler.
            float rb0 = 0.f, rb1 = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint32_t w0 = pack_bf16x2(p[8 * ks + 0], p[8 * ks + 1]);
                const uint32_t w1 = pack_bf16x2(p[8 * ks + 2], p[8 * ks + 3]);
                const uint32_t w2 = pack_bf16x2(p[8 * ks + 4], p[8 * ks + 5]);
                const uint32_t w3 = pack_bf16x2(p[8 * ks + 6], p[8 * ks + 7]);
                rb0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), kOnes, rb0, false);
                rb1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), kOnes, rb1, false);
                rb0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), kOnes, rb0, false);
                rb1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), kOnes, rb1, false);
                const u32x4 w = {w0, w1, w2, w3};
                pbo[ks] = __builtin_bit_cast(bf16x8, w);
            }
            rs = rs0 + rs1;
            rb = rb0 + rb1;
        };

        // One 32-key pipeline step (block k): the softmax of block k on the VALU
        // interleaves with the matrix-core work of the scores of block k+1 (K rows
        // from byte kq of buffer kbuf) and P V of block k-1 (V rows from byte vp of
        // buffer vbuf).  The first step multiplies the zeroed V buffer by P = 0;
        // the last computes scores of a block that does not exist and discards
        // them.  MASKED steps apply the causal / sequence-end mask.  LOADS steps
        // also copy K tile load_t+1 into kdst and V tile load_t into vdst, spread
        // among their MFMAs.
        auto step = [&](int k, const char *kbuf, int kq, const char *vbuf, int vp, auto masked_tag,
                        auto next_masked_tag, auto loads_tag, int load_t, char *kdst, char *vdst) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            constexpr bool NEXT_MASKED = decltype(next_masked_tag)::value;
            constexpr bool LOADS = decltype(loads_tag)::value;
            // Keep the per-lane LDS offsets opaque inside the loop: otherwise
            // their sums with each buffer's constant base are hoisted out of the
            // loop as separate registers instead of riding in the ds_read
            // immediate offset field.
#pragma unroll
            for (int st = 0; st < T::kQkSteps; ++st)
                asm volatile("" : "+v"(koff[st]));
#pragma unroll
            for (int b = 0; b < T::kOBlocks; ++b)
                asm volatile("" : "+v"(voff[b][0]), "+v"(voff[b][1]));
            // Pin the softmax inside its step: without this, loop rotation moves
            // the first step's VALU work into the previous iteration's latch, away
            // from the MFMAs it is meant to overlap.
            asm volatile("" : "+v"(sc));

            // This block's P is taken against m_sub (the reference max, log2
            // units), fixed before the step, so the exps need nothing from this
            // block's max.  d = 128: the previous step checked that every
            // visible p stays <= 2^kRefSlack.  d = 64: this step checks its own
            // sums after the exps and, in the rare case, takes the block again.
            // l sums the fp32 p (for the LSE), lb the bf16-rounded p that P V
            // actually multiplies (for O).
            bf16x8 pb[2];
            float rs, rb;
            block_softmax(sc, m_sub, k, masked_tag, pb, rs, rb);
            if constexpr (!kSumCheck) {
                l_run += rs;
                lb_run += rb;
            }

            if constexpr (LOADS) {
                load_tile(Kh, (load_t + 1) * kBc, kdst, kdma);
                load_tile(Vh, load_t * kBc, vdst, vdma);
            }
            f32x16 sn = {};
#pragma unroll
            for (int st = 0; st < T::kQkSteps; ++st)
                sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*LDS_PTR(const bf16x8, kbuf + kq + koff[st]), qop[st],
                                                             sn, 0, 0, 0);
            pv(vbuf, vp, pb_prev);

            // d = 128: row max of the next block (this lane's half of its keys,
            // log2 units), for the next step's reference.  d = 64: whether some
            // lane's sum of this block passed kSumLimit (inf included).
            float mx = kNegInf;
            bool reref = false;
            if constexpr (kSumCheck) {
                reref = __builtin_amdgcn_ballot_w64(rs > kSumLimit) != 0;  // wave-uniform
            } else {
                if constexpr (NEXT_MASKED) {
                    mx = kNegInf;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        mx = fmaxf(mx, visible(k + 1, r) ? sn[r] * c_log2 : kNegInf);
                } else {  // every key visible and c_log2 > 0
                    float r0 = sn[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r)
                        r0 = fmaxf(r0, sn[r]);
                    mx = r0 * c_log2;
                }
                reref = __builtin_amdgcn_ballot_w64(mx > m_thr) != 0;  // wave-uniform
            }

            // Issue order for this step's scheduling region: the 16 MFMAs (8 for
            // the next scores, 8 for P V) each followed by the operand reads two
            // MFMAs ahead (8 ds_read_b128 of K, 16 ds_read_b64_tr_b16 of V in
            // all, hiding LDS latency with a bounded number of registers in
            // flight) and then a share of the softmax VALU work, so the matrix
            // cores and the VALU stay busy together.  Reads before the VALU
            // share measured 1% faster than after it.
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
#pragma unroll
            for (int i = 0; i < 2 * T::kQkSteps; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
                __builtin_amdgcn_sched_group_barrier(0x402, kValuPerMfma, 0);  // VALU incl. transcendental
                if (LOADS && i < 2 * T::kLoadsPerWave)
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // tile copy (VMEM)
            }
            // Keep this block's P and row sums inside this step: otherwise the
            // compiler sinks the exps and adds next to their first uses (the next
            // step's P V and the loop latch), where no MFMA is left to hide them.
            if constexpr (kSumCheck)
                asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(rs), "+v"(rb));
            else
                asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(l_run), "+v"(lb_run));

            if constexpr (kSumCheck) {
                // Some lane's probabilities of this block passed kSumLimit against
                // the reference: move the reference to the row's exact running max
                // (this block's scores are still in registers), rescale l, lb and
                // O (which now holds P V up to block k-1, all against the old
                // reference), and take this block's probabilities again.  (Rare:
                // laid out off the step's straight line.)
                if (__builtin_expect(reref, 0)) {
                    float mb = kNegInf;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float t = sc[r] * c_log2;
                        mb = fmaxf(mb, (!MASKED || visible(k, r)) ? t : kNegInf);
                    }
                    const float m_new = fmaxf(m_ref, wave_half_max(mb));
                    const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                    l_run *= alpha;
                    lb_run *= alpha;
#pragma unroll
                    for (int b = 0; b < T::kOBlocks; ++b)
                        oacc[b] *= alpha;
                    set_ref(m_new);
                    block_softmax(sc, m_sub, k, masked_tag, pb, rs, rb);
                }
                l_run += rs;
                lb_run += rb;
            } else {
                // The reference moved at the previous step: O now holds P V of
                // block k-1 as well, taken against the old reference, so rescale
                // it here.  (Both branches are rare: laid out off the step's
                // straight line.)
                if (__builtin_expect(pending, 0)) {
#pragma unroll
                    for (int b = 0; b < T::kOBlocks; ++b)
                        oacc[b] *= alpha_pend;
                }
                // Some row of the next block has a p above 2^kRefSlack against the
                // current reference: move the reference to the row's exact running
                // max (both halves of the row) and rescale the sums now, O after
                // the next P V.
                pending = reref;
                if (__builtin_expect(reref, 0)) {
                    const float m_new = fmaxf(m_ref, wave_half_max(mx));
                    alpha_pend = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                    l_run *= alpha_pend;
                    lb_run *= alpha_pend;
                    set_ref(m_new);
                }
            }
            sc = sn;
            pb_prev[0] = pb[0];
            pb_prev[1] = pb[1];
        };

        // One 64-key tile t held in K buffer P = t % 2 (V tile t-1 in V buffer
        // 1-P).  The even step makes the last reads of K tile t and V tile t-1;
        // after the barrier the odd step refills those buffers with K tile t+2 and
        // V tile t+1 (past the end: zeros, no memory traffic), which land before
        // the next barrier.
        // NEXT_MASKED: whether the block after the tile (the first of tile t+1)
        // needs the mask.
        auto tile = [&](int t, auto parity_tag, auto masked_tag, auto next_masked_tag) __attribute__((always_inline)) {
            constexpr int P = decltype(parity_tag)::value;
            constexpr int kHalf = 32 * T::kRowBytes;
            char *kp = P ? sk1 : sk0, *kq = P ? sk0 : sk1;
            char *vp = P ? sv1 : sv0, *vq = P ? sv0 : sv1;
            step(2 * t, kp, kHalf, vq, kHalf, masked_tag, masked_tag, std::false_type{}, 0, kp, vq);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            step(2 * t + 1, kq, 0, vp, 0, masked_tag, next_masked_tag, std::true_type{}, t + 1, kp, vq);
        };
        // A tile whose every step is dead for this wave under the causal mask:
        // P V of its first step's block 2t-1 and everything after start past
        // the wave's last query.  The wave still copies its share of the
        // tiles and meets the barrier, so the other waves see no difference.
        const int last_live = (qw0 + kRowsPerWave - 1 + delta) / 32;  // last 32-key block with a visible key
        auto dead = [&](int t) __attribute__((always_inline)) { return CAUSAL && 2 * t - 1 > last_live; };
        auto ghost = [&](int t, auto parity_tag) __attribute__((always_inline)) {
            constexpr int P = decltype(parity_tag)::value;
            char *kp = P ? sk1 : sk0;
            char *vq = P ? sv0 : sv1;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            load_tile(Kh, (t + 2) * kBc, kp, kdma);
            load_tile(Vh, (t + 1) * kBc, vq, vdma);
        };
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using Unmasked = std::false_type;
        using Masked = std::true_type;

        // In the tiles that need the mask for some query of the workgroup, each
        // step picks its code for this wave alone: a 32-key block whose every
        // key is visible to all 32 queries of the wave (below the wave's own
        // diagonal and inside the key range) needs neither the masked exps nor
        // the masked row max (which also asks for a positive scale), so only
        // the blocks that cross the wave's diagonal or the range end pay for
        // the mask.  The choice is wave-uniform.
        const int vis_lim = c_log2 > 0.f ? min(CAUSAL ? qw0 + delta : 0x7fffffff, kv_hi - 1) : -1;
        auto full = [&](int kb) __attribute__((always_inline)) { return 32 * kb + 31 <= vis_lim; };
        auto mstep = [&](int k, const char *kbuf, int kq, const char *vbuf, int vp, auto loads_tag, int load_t,
                         char *kdst, char *vdst) __attribute__((always_inline)) {
            if constexpr (kSumCheck) {  // the next block's mask matters only to the row-max guard
                if (full(k))
                    step(k, kbuf, kq, vbuf, vp, Unmasked{}, Unmasked{}, loads_tag, load_t, kdst, vdst);
                else
                    step(k, kbuf, kq, vbuf, vp, Masked{}, Masked{}, loads_tag, load_t, kdst, vdst);
            } else if (full(k + 1))
                step(k, kbuf, kq, vbuf, vp, Unmasked{}, Unmasked{}, loads_tag, load_t, kdst, vdst);
            else if (full(k))
                step(k, kbuf, kq, vbuf, vp, Unmasked{}, Masked{}, loads_tag, load_t, kdst, vdst);
            else
                step(k, kbuf, kq, vbuf, vp, Masked{}, Masked{}, loads_tag, load_t, kdst, vdst);
        };
        // A masked tile.  Under the causal mask its odd step is dead for this
        // wave when block 2t, the one whose P V that step takes, is already past
        // the wave's last visible key: block 2t then has p = 0 everywhere, the
        // step would add nothing to O, l or lb, and no row can move its
        // reference (its sums are 0).  The wave then only makes the step's
        // copies, and every later tile is dead for it as well.
        auto tile_m = [&](int t, auto parity_tag) __attribute__((always_inline)) {
            constexpr int P = decltype(parity_tag)::value;
            constexpr int kHalf = 32 * T::kRowBytes;
            char *kp = P ? sk1 : sk0, *kq = P ? sk0 : sk1;
            char *vp = P ? sv1 : sv0, *vq = P ? sv0 : sv1;
            mstep(2 * t, kp, kHalf, vq, kHalf, std::false_type{}, 0, kp, vq);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (CAUSAL && 2 * t > last_live) {
                load_tile(Kh, (t + 2) * kBc, kp, kdma);
                load_tile(Vh, (t + 1) * kBc, vq, vdma);
            } else {
                mstep(2 * t + 1, kq, 0, vp, 0, std::true_type{}, t + 1, kp, vq);
            }
        };

        // Tiles [t_lo, t_free) need no mask: inside the key range and below the
        // causal diagonal of every query of the workgroup (and a positive scale,
        // which the unmasked row max assumes).  t_free - t_lo is made even so
        // that the loops walk (buffer 0, buffer 1) tile pairs (t_lo is even);
        // the last unmasked pair is peeled because the block after it needs the
        // mask.
        int t_free = kv_hi / kBc;
        if (CAUSAL)
            t_free = min(t_free, (q0 + delta + 1) / kBc);
        if (!(c_log2 > 0.f))
            t_free = t_lo;
        t_free = max(t_lo, min(t_free, t_end));
        t_free = t_lo + ((t_free - t_lo) & ~1);
        int t = t_lo;
        if (qw0 >= Nq) {
            // No query of this wave exists: copy its share of every tile and
            // meet every barrier, nothing else.
            for (; t < t_end; t += 2) {
                ghost(t, P0{});
                if (t + 1 < t_end)
                    ghost(t + 1, P1{});
            }
        } else {
            for (; t + 2 < t_free; t += 2) {
                tile(t, P0{}, Unmasked{}, Unmasked{});
                tile(t + 1, P1{}, Unmasked{}, Unmasked{});
            }
            if (t < t_free) {
                tile(t, P0{}, Unmasked{}, Unmasked{});
                tile(t + 1, P1{}, Unmasked{}, Masked{});
                t += 2;
            }
            // (Without the causal mask only a ragged end is masked: those tiles
            // keep the one masked step code.  So does the 4-wave d = 128 decoding
            // instance, whose masked tiles are at most the last one or two of a
            // key range: with the per-wave choice the compiler kept its masked
            // step in source order.)
            constexpr bool kPerWaveMask = CAUSAL && !(D == 128 && W == 4);
            for (; t < t_end; t += 2) {
                if (dead(t))
                    ghost(t, P0{});
                else if constexpr (kPerWaveMask)
                    tile_m(t, P0{});
                else
                    tile(t, P0{}, Masked{}, Masked{});
                if (t + 1 < t_end) {
                    if (dead(t + 1))
                        ghost(t + 1, P1{});
                    else if constexpr (kPerWaveMask)
                        tile_m(t + 1, P1{});
                    else
                        tile(t + 1, P1{}, Masked{}, Masked{});
                }
            }
            // P V of the last block: second half of V tile t_end-1.
            pv((t_end - 1) & 1 ? sv1 : sv0, 32 * T::kRowBytes, pb_prev);
            if (__builtin_expect(pending, 0)) {
#pragma unroll
                for (int b = 0; b < T::kOBlocks; ++b)
                    oacc[b] *= alpha_pend;
            }
        }
        // O is read only by the lanes of valid queries: keep its MFMAs out of
        // that lane-masked branch (an MFMA under a partial EXEC mask does not
        // compute the lanes' tile).
#pragma unroll
        for (int b = 0; b < T::kOBlocks; ++b)
            asm volatile("" : "+v"(oacc[b]));
        __builtin_amdgcn_s_waitcnt(0);  // no copy may still be writing LDS when the workgroup ends

        // Epilogue: O = O / lb (the sum of the bf16 weights that built O),
        // LSE = ln2 * (m + log2 l) from the fp32 sum.  In a key range where a
        // row sees no key (split mode only) l = lb = 0: LSE = -inf, O = 0.
        const float l_tot = wave_half_sum(l_run);
        const float lb_tot = wave_half_sum(lb_run);
        if (q_ok) {
            const float inv = lb_tot > 0.f ? 1.f / lb_tot : 0.f;
            const float lse = (m_ref + __builtin_log2f(l_tot)) * 0.69314718055994530942f;
            if constexpr (SPLIT) {
                float *op = a.Opart + (((size_t)split * a.BH + bh) * Nq + qidx) * D;
#pragma unroll
                for (int b = 0; b < T::kOBlocks; ++b)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<f32x4 *>(op + 32 * b + 8 * j + 4 * half) =
                            f32x4{oacc[b][4 * j + 0] * inv, oacc[b][4 * j + 1] * inv, oacc[b][4 * j + 2] * inv,
                                  oacc[b][4 * j + 3] * inv};
                if (half == 0)
                    a.LSEpart[((size_t)split * a.BH + bh) * Nq + qidx] = l_tot > 0.f ? lse : kNegInf;
            } else {
                __bf16 *orow = a.O + qhead + (size_t)qidx * D;
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
                if (a.LSE != nullptr && half == 0)
                    a.LSE[(size_t)bh * Nq + qidx] = lse;
            }
        }
    }
#endif
}

// Merge of the split ranges (the two-block merge equation of "FlashAttention
// evolution", letsgetai.github.io, core-mechanism section, applied to S
// blocks): LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.  One
// thread per 8 head-dim columns of one query row; memory-bound (it reads
// S (4 d + 4) bytes and writes 2 d + 4 bytes per row), so it is laid out for
// 16-byte coalesced loads and stores and nothing else.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float *__restrict__ Opart,
                                                        const float *__restrict__ LSEpart,
                                                        __bf16 *__restrict__ O, float *__restrict__ LSE,
                                                        int rows, int S)
{
    constexpr int kChunks = D / 8;
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    const int row = gid / kChunks, c = gid % kChunks;
    if (row >= rows)
        return;
    float m = kNegInf;
    for (int s = 0; s < S; ++s)
        m = fmaxf(m, LSEpart[(size_t)s * rows + row]);
    f32x4 acc0 = {}, acc1 = {};
    float wsum = 0.f;
    if (m != kNegInf) {
        for (int s = 0; s < S; ++s) {
            const float ls = LSEpart[(size_t)s * rows + row];
            const float w = __builtin_amdgcn_exp2f((ls - m) * kLog2e);  // 0 for an empty range
            const float *src = Opart + ((size_t)s * rows + row) * D + 8 * c;
            acc0 += w * *reinterpret_cast<const f32x4 *>(src);
            acc1 += w * *reinterpret_cast<const f32x4 *>(src + 4);
            wsum += w;
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    u32x4 out;
    out[0] = pack_bf16x2(acc0[0] * inv, acc0[1] * inv);
    out[1] = pack_bf16x2(acc0[2] * inv, acc0[3] * inv);
    out[2] = pack_bf16x2(acc1[0] * inv, acc1[1] * inv);
    out[3] = pack_bf16x2(acc1[2] * inv, acc1[3] * inv);
    *reinterpret_cast<u32x4 *>(O + (size_t)row * D + 8 * c) = out;
    if (LSE != nullptr && c == 0)
        LSE[row] = wsum > 0.f ? m + __builtin_logf(wsum) : kNegInf;
}

// The merge of the key ranges in the split workspace into O and LSE.
template <int D>
static hipError_t merge_launch(const AttnLaunch &a, int splits)
{
    const float *opart = (const float *)a.workspace;
    const float *lsepart = opart + (size_t)splits * a.BH * a.Nq * D;
    const int rows = (int)(a.BH * a.Nq);
    const int threads = rows * (D / 8);
    hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((threads + 255) / 256), dim3(256), 0, a.stream, opart, lsepart,
                       (__bf16 *)a.o, a.lse, rows, splits);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPLIT, int W = Tile<D>::kWaves>
static hipError_t launch(const AttnLaunch &a, int splits, int split_keys)
{
    using T = Tile<D, W>;
    KArgs k;
    k.Q = (const __bf16 *)a.q;
    k.K = (const __bf16 *)a.k;
    k.V = (const __bf16 *)a.v;
    k.O = (__bf16 *)a.o;
    k.LSE = a.lse;
    k.Opart = SPLIT ? (float *)a.workspace : nullptr;
    k.LSEpart = SPLIT ? (float *)a.workspace + (size_t)splits * a.BH * a.Nq * D : nullptr;
    k.BH = (int)a.BH;
    k.Nq = (int)a.Nq;
    k.Nk = (int)a.Nk;
    k.nqt = (int)((a.Nq + T::kBr - 1) / T::kBr);
    k.n_splits = splits;
    k.split_keys = split_keys;
    // Causal, one key range: pairs of query tiles, or single tiles longest
    // first when the pairs would not fill the chip's workgroup slots twice
    // (256 CUs, 4 SIMDs x waves_per_simd / W workgroups each) and the heads
    // split evenly over the XCDs.
    const int64_t pairs = a.BH * ((k.nqt + 1) / 2);
    const int64_t slots = 256 * (4 * waves_per_simd<D>() / W);
    k.lpt = CAUSAL && !SPLIT && a.BH % kXcds == 0 && pairs < 2 * slots;
    k.n_wg = (int)(a.BH * ((CAUSAL && !k.lpt) ? (k.nqt + 1) / 2 : k.nqt) * splits);
    k.c_log2 = a.scale * kLog2e;
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, SPLIT, W>), dim3(k.n_wg), dim3(T::kThreads), 0, a.stream, k);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || !SPLIT)
        return err;
    return merge_launch<D>(a, splits);
}

template <int D, bool CAUSAL>
static hipError_t launch_mode(const AttnLaunch &a)
{
    const int64_t splits = attn_splits_used(a.Nk, a.num_splits);
    if (splits <= 1)
        return launch<D, CAUSAL, false>(a, 1, (int)attn_split_keys(a.Nk, 1));
    if (a.Nq <= kDecodeRows) {  // a few query rows: the streaming kernel, then the merge
        const hipError_t err = attn_decode_ranges_launch(a, (int)splits, (int)attn_split_keys(a.Nk, a.num_splits));
        if (err != hipSuccess)
            return err;
        return merge_launch<D>(a, (int)splits);
    }
    if constexpr (D == 128) {
        if (a.Nq <= 128)  // decoding: one 4-wave query tile per head and range
            return launch<D, CAUSAL, true, 4>(a, (int)splits, (int)attn_split_keys(a.Nk, a.num_splits));
    }
    return launch<D, CAUSAL, true>(a, (int)splits, (int)attn_split_keys(a.Nk, a.num_splits));
}

}  // namespace attn_gfx950

int64_t attn_split_keys(int64_t Nk, int64_t num_splits)
{
    // ceil(Nk / num_splits) rounded up to two 64-key tiles, so every range
    // starts on an even tile
    const int64_t per = (Nk + num_splits - 1) / num_splits;
    return ((per + 127) / 128) * 128;
}

int64_t attn_splits_used(int64_t Nk, int64_t num_splits)
{
    const int64_t keys = attn_split_keys(Nk, num_splits);
    return keys > 0 ? (Nk + keys - 1) / keys : 1;
}

int64_t attn_splitkv_workspace_bytes(int64_t BH, int64_t Nq, int64_t d, int64_t num_splits)
{
    return num_splits * BH * Nq * (d + 1) * 4;
}

int64_t attn_workgroups(int64_t BH, int64_t Nq, int64_t Nk, int64_t num_splits)
{
    // An upper bound over head dims and masks: the smallest query tile.
    return BH * ((Nq + attn_gfx950::kBrMin - 1) / attn_gfx950::kBrMin) * attn_splits_used(Nk, num_splits);
}

hipError_t attn_launch(const AttnLaunch &a)
{
    using namespace attn_gfx950;
    if (a.d == 128)
        return a.causal ? launch_mode<128, true>(a) : launch_mode<128, false>(a);
    return a.causal ? launch_mode<64, true>(a) : launch_mode<64, false>(a);
}
