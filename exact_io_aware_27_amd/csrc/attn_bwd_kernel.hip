// attn_bwd_kernel.hip -- gradients of exact attention for gfx950 (the
// backward pass), by recomputation.
//
// The forward pass keeps only O and the per-row logsumexp; the backward pass
// recomputes the scores and probabilities tile by tile from them instead of
// reading an N x N matrix back ("FlashAttention evolution",
// letsgetai.github.io, recomputation paragraph; "FlashAttention" concept
// page, compassingai.com, section 3).  With P_ij = exp(scale q_i.k_j - LSE_i)
// and an upstream gradient dO:
//
//   D_i   = dO_i . O_i
//   dS_ij = P_ij (dO_i . v_j - D_i)
//   dV_j  = sum_i P_ij dO_i,   dK_j = scale sum_i dS_ij q_i,   dQ_i = scale sum_j dS_ij k_j
//
// Two kernels, each owning what it writes, so nothing is accumulated with
// atomics and every result is deterministic:
//   * attn_bwd_dq_kernel walks the keys of a query tile (the forward loop
//     order).  It computes D and the LSE in log2 units for its rows, stores
//     both for the second kernel, and accumulates dQ.
//   * attn_bwd_dkdv_kernel walks the queries of a key tile and accumulates
//     dK and dV.
// The scores S and dP = dO V^T are computed in both (seven 32x32-block
// matrix products per block pair in all, against five when dQ is summed with
// atomics); in exchange there is no atomic traffic and no dQ workspace.
//
// gfx950 mapping (shared by both kernels)
//   * 32 rows (queries or keys) per wave; 8 waves per workgroup for d = 128
//     (one workgroup per CU), 4 for d = 64 (two per CU).  Each lane owns one
//     row of its wave (lane % 32) in the 32x32 accumulator layout of
//     v_mfma_f32_32x32x16_bf16 and 16 of the 32 columns of the other side.
//   * The operands walked by the loop (K and V in the dQ kernel, Q and dO in
//     the dK/dV kernel) go from global memory to LDS in 64-row tiles with
//     buffer_load_dwordx4 ... lds, double-buffered, one barrier per tile;
//     tiles are walked in (buffer 0, buffer 1) pairs so that every LDS
//     address is a constant plus a per-lane offset.  Rows past N read as
//     zeros, with no memory access.
//   * Each tile is read both row-wise (ds_read_b128, as the A operand of a
//     product over the head dim) and transposed (ds_read_b64_tr_b16, as the
//     A operand of a product over the rows), so one XOR swizzle of 16-byte
//     chunks serves both: conflict-free for 16 consecutive rows at one chunk
//     and for 4 aligned rows times one 32-column block.
//   * The probabilities and dS leave the score accumulator in the register
//     order of the B operand of the next product; the transposed reads use
//     the matching row order, so nothing is shuffled in registers.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn_gfx950 {
namespace bwd {

constexpr int kRows = 32;     // rows per wave
constexpr int kBlockMin = 128;  // fewest rows (queries or keys) a workgroup owns
constexpr int kTile = 64;     // rows per LDS tile of the walked operands

// Workgroup shape per head dim, as in the forward pass: d = 128 runs 8 waves
// (one workgroup per CU), so each tile copied into LDS serves 256 rows; d = 64
// runs 4 waves, two workgroups per CU.  Either way two waves share a SIMD.
template <int D>
struct Shape {
    static constexpr int kWaves = D == 128 ? 8 : 4;
    static constexpr int kThreads = kWave * kWaves;
    static constexpr int kBlock = kRows * kWaves;         // rows a workgroup owns
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
    static constexpr int kBytes = kTile * kRowBytes;      // one tile
    static constexpr int kSteps = D / 16;                 // MFMA k-steps over the head dim
    static constexpr int kDBlocks = D / 32;               // 32-row blocks of a d x 32 accumulator
    static constexpr int kRowsPerLoad = 1024 / kRowBytes; // rows one wave-wide 16-byte load fills
    static constexpr int kLoadsPerWave = kBytes / 1024 / kWaves;
};

// Chunk c of tile row r sits at chunk position c ^ swz(r).
//  Row reads: lanes 0..15 read rows 0..15 (mod 16) at one chunk; the LDS
//  serves 16 such 16-byte reads per cycle, so the 16 positions (with the
//  row's place in its 256-byte bank line) must differ.
//  Transposed reads: 32 lanes read 4 aligned rows times the 4 chunks of one
//  32-column block, 8 bytes each; the 4 rows must land on distinct 64-byte
//  bank blocks.
//  d = 128 (one row per bank line): bits 2..3 from r & 3 (transposed reads),
//  bits 0..1 from (r >> 2) & 3 (with them, 16 distinct values).
//  d = 64 (two rows per bank line, parity picks the half): bit 2 from
//  (r >> 1) & 1 separates rows r and r + 2, bits 0..1 from (r >> 2) & 3.
template <int D>
__device__ __forceinline__ int swz(int r)
{
    if constexpr (D == 128)
        return ((r & 3) << 2) | ((r >> 2) & 3);
    else
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D>
__device__ __forceinline__ uint32_t lds_off(int r, int c)
{
    return (uint32_t)(r * Shape<D>::kRowBytes + ((c ^ swz<D>(r)) << 4));
}

// Kernel arguments.  Q, O, dO, dQ: [BH][N][d]; K, V, dK, dV: [BH][N][d];
// LSE: [BH][N] (natural log, from the forward pass).  L2 and Dsum, [BH][N]
// each, are written by the dQ kernel and read by the dK/dV kernel: the LSE in
// log2 units and -D.  c_log2 = scale * log2(e).
struct BArgs {
    const __bf16 *Q, *K, *V, *O, *dO;
    const float *LSE;
    float *L2, *Dsum;
    __bf16 *dQ, *dK, *dV;
    int BH, N, n_wg, ntiles;
    int lpt;  // causal: single blocks, longest first (see block_of)
    float c_log2, scale;
};

// Per-lane LDS offsets of one tile, fixed for the whole loop.
template <int D>
struct Offsets {
    using S = Shape<D>;
    uint32_t dma[S::kLoadsPerWave];  // global byte offset (within a tile) this lane copies
    uint32_t row[S::kSteps];         // row read: row n of a 32-row block, chunk 2 st + half
    uint32_t tr[S::kDBlocks][2];     // transposed read: see below

    __device__ __forceinline__ Offsets(int wave, int lane)
    {
        const int n = lane & 31, half = lane >> 5;
#pragma unroll
        for (int i = 0; i < S::kLoadsPerWave; ++i) {
            const int slice = wave * S::kLoadsPerWave + i;
            const int r = slice * S::kRowsPerLoad + lane / S::kChunks;
            const int pos = lane % S::kChunks;
            dma[i] = (uint32_t)(r * S::kRowBytes + ((pos ^ swz<D>(r)) << 4));
        }
#pragma unroll
        for (int st = 0; st < S::kSteps; ++st)
            row[st] = lds_off<D>(n, 2 * st + half);
        // ds_read_b64_tr_b16 within a 16-lane group g hands lane j element j % 4
        // of source lanes j / 4 + 4 e.  Source lane i of group g reads row
        // 8 jj + 4 (g / 2) + i / 4 of a 16-row step, head-dim columns
        // 32 b + 16 (g % 2) + 4 (i % 4) .. +3, so lane l = 16 g + j receives
        // column 32 b + l % 32 of rows 8 jj + 4 (l / 32) + e: the A operand of
        // a product over the rows, in the row order the score accumulator
        // hands its B operand (register 4 j + e of a lane in half h holds row
        // 8 j + 4 h + e).
        const int g = lane >> 4, i = lane & 15;
#pragma unroll
        for (int b = 0; b < S::kDBlocks; ++b)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int r = 8 * jj + 4 * (g >> 1) + (i >> 2);
                const int dcol = 32 * b + 16 * (g & 1) + 4 * (i & 3);
                tr[b][jj] = lds_off<D>(r, dcol >> 3) + ((dcol & 4) << 1);
            }
    }

    // Make the offsets opaque to the optimiser at the start of a tile, so that
    // their sums with each buffer's constant base are not hoisted out of the
    // loop as separate registers instead of riding in the LDS read offset.
    __device__ __forceinline__ void opaque()
    {
#pragma unroll
        for (int st = 0; st < S::kSteps; ++st)
            asm volatile("" : "+v"(row[st]));
#pragma unroll
        for (int b = 0; b < S::kDBlocks; ++b)
            asm volatile("" : "+v"(tr[b][0]), "+v"(tr[b][1]));
    }
};

// One 64-row tile of a [N][d] operand of head `src` (rows from row0) into an
// LDS buffer: this wave's slices, one buffer_load_dwordx4 ... lds each.
// Rows at or past `rows` (the head's N) read as zeros with no memory access.
template <int D>
__device__ __forceinline__ void load_tile(const __bf16 *src, int rows, int row0, char *buf, int wave_u,
                                          const uint32_t *dma)
{
    using S = Shape<D>;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, (int)((uint32_t)rows * S::kRowBytes), kBufferFlags);
#pragma unroll
    for (int i = 0; i < S::kLoadsPerWave; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, buf + (wave_u * S::kLoadsPerWave + i) * 1024), 16,
                                                 dma[i], (int)((uint32_t)row0 * (uint32_t)S::kRowBytes), 0, 0);
}

// 64 floats of a [N] row vector (from row0) into LDS, by one wave: one
// 4-byte buffer_load ... lds.  Entries past N read as zero.
__device__ __forceinline__ void load_vec(const float *src, int rows, int row0, float *buf, int lane)
{
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, (int)((uint32_t)rows * 4u), kBufferFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, buf), 4, (uint32_t)lane * 4u,
                                             (int)((uint32_t)row0 * 4u), 0, 0);
}

// C (32 rows x 32 columns) = init + A B over the head dim: A rows from LDS
// at `base` (row read offsets), B operand resident in registers.
template <int D>
__device__ __forceinline__ f32x16 rows_times(const char *base, const Offsets<D> &off, const bf16x8 *bop,
                                             const f32x16 &init = f32x16{})
{
    f32x16 c = init;
#pragma unroll
    for (int st = 0; st < Shape<D>::kSteps; ++st)
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*LDS_PTR(const bf16x8, base + off.row[st]), bop[st], c, 0, 0, 0);
    return c;
}

// acc[b] (d x 32) += X^T W over the 32 rows of a block: X^T through the
// transposed reads of the tile rows at `base`, W the packed B operand (two
// 16-row k-steps).
template <int D>
__device__ __forceinline__ void tr_times(f32x16 *acc, const char *base, const Offsets<D> &off, const bf16x8 *w)
{
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int b = 0; b < Shape<D>::kDBlocks; ++b) {
            const char *p = base + ks * 16 * Shape<D>::kRowBytes;
            const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                           LDS_PTR(s16x4, p + off.tr[b][0])));
            const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                           LDS_PTR(s16x4, p + off.tr[b][1])));
            const u32x4 xa = {lo[0], lo[1], hi[0], hi[1]};
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa), w[ks], acc[b], 0, 0, 0);
        }
}

// 16 fp32 values of one lane's score-layout registers as the two bf16x8 B
// operands of a product over those rows (registers 8 ks .. 8 ks + 7).
__device__ __forceinline__ void pack_b(const float *x, bf16x8 *w)
{
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const u32x4 u = {pack_bf16x2(x[8 * ks + 0], x[8 * ks + 1]), pack_bf16x2(x[8 * ks + 2], x[8 * ks + 3]),
                         pack_bf16x2(x[8 * ks + 4], x[8 * ks + 5]), pack_bf16x2(x[8 * ks + 6], x[8 * ks + 7])};
        w[ks] = __builtin_bit_cast(bf16x8, u);
    }
}

// 8 bf16 of row `row` (zeros when !ok), columns col .. col+7.
__device__ __forceinline__ bf16x8 row8(const __bf16 *base, int row, bool ok, int col, int D)
{
    if (!ok)
        return bf16x8{};
    return *reinterpret_cast<const bf16x8 *>(base + (size_t)row * D + col);
}

// Store a d x 32 accumulator (rows = head dim, column = this lane's row of
// the output) times `mul` as bf16 into out[row][*].
template <int D>
__device__ __forceinline__ void store_rows(__bf16 *out_row, const f32x16 *acc, float mul, int half)
{
#pragma unroll
    for (int b = 0; b < Shape<D>::kDBlocks; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[b][4 * j + 0] * mul, acc[b][4 * j + 1] * mul);
            w[1] = pack_bf16x2(acc[b][4 * j + 2] * mul, acc[b][4 * j + 3] * mul);
            *reinterpret_cast<u32x2 *>(out_row + 32 * b + 8 * j + 4 * half) = w;
        }
}

// Causal load balance: a workgroup runs block nblk-1-u and then block u of
// one head (the middle block of an odd count alone), so every workgroup walks
// nearly the same number of tiles.
__device__ __forceinline__ int pair_block(bool causal, int nblk, int unit, int pass)
{
    return causal ? (pass == 0 ? nblk - 1 - unit : unit) : unit;
}

// Workgroup -> (head, unit, passes).  A causal grid too small to fill the
// chip twice over with pairs runs single blocks instead, longest first within
// each XCD: XCD x owns heads [x B H / 8, (x + 1) B H / 8) (the host chooses
// this only when 8 divides B H), and its workgroups walk them block by block
// from the heaviest; unit r is then the r-th heaviest block, which
// heavy_block turns into a block index.
__device__ __forceinline__ void block_of(const BArgs &a, int nblk, bool causal, int &bh, int &unit, int &npass)
{
    if (causal && a.lpt) {
        const int hpx = a.BH / kXcds, xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
        bh = xcd * hpx + slot % hpx;
        unit = slot / hpx;
        npass = 1;
        return;
    }
    const int n_units = causal ? (nblk + 1) / 2 : nblk;
    unit_of(blockIdx.x, a.n_wg, n_units, bh, unit);
    npass = (causal && nblk - 1 - unit != unit) ? 2 : 1;
}

// ---------------------------------------------------------------------------
// dQ (and D, L2): one workgroup per query block of one head.  Per 32-key
// block: S^T = K Q^T and dP^T = V dO^T (keys x queries), P^T = exp2(S^T
// c_log2 - L2), dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(Shape<D>::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dq_kernel(
    const BArgs a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using S = Shape<D>;
    __shared__ __attribute__((aligned(1024))) char sk0[S::kBytes];
    __shared__ __attribute__((aligned(1024))) char sk1[S::kBytes];
    __shared__ __attribute__((aligned(1024))) char sv0[S::kBytes];
    __shared__ __attribute__((aligned(1024))) char sv1[S::kBytes];

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave_u = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int n = lane & 31, half = lane >> 5;
    const int N = a.N, nblk = a.ntiles;

    int bh, unit, npass;
    block_of(a, nblk, CAUSAL, bh, unit, npass);
    const size_t head = (size_t)bh * (size_t)N * D;
    const __bf16 *Kh = a.K + head, *Vh = a.V + head;

    for (int pass = 0; pass < npass; ++pass) {
        // Per-lane LDS offsets, built afresh in each pass from an opaque copy of
        // the lane index so that they are not held live across passes.
        int lane_p = lane;
        asm volatile("" : "+v"(lane_p));
        Offsets<D> off(wave_u, lane_p);
        if (pass > 0)
            __syncthreads();  // every wave is done with the previous block's LDS
        // (longest first: the heaviest query block is the last)
        const int q0 = (CAUSAL && a.lpt ? nblk - 1 - unit : pair_block(CAUSAL, nblk, unit, pass)) * S::kBlock;
        const int qw0 = q0 + wave_u * kRows;
        const int qidx = qw0 + n;
        const bool q_ok = qidx < N;
        const bool wave_live = qw0 < N;
        const int kv_end = CAUSAL ? min(N, q0 + S::kBlock) : N;
        const int t_end = (kv_end + kTile - 1) / kTile;

        load_tile<D>(Kh, kv_end, 0, sk0, wave_u, off.dma);
        load_tile<D>(Vh, kv_end, 0, sv0, wave_u, off.dma);

        // Q^T and dO^T operands, resident: k-step st holds columns
        // 16 st + 8 half .. +7 of this lane's query row.  D = dO . O from the
        // same columns, summed over both halves.
        bf16x8 qop[S::kSteps], gop[S::kSteps];
        float dpart = 0.f;
#pragma unroll
        for (int st = 0; st < S::kSteps; ++st) {
            const int col = 16 * st + 8 * half;
            qop[st] = row8(a.Q + head, qidx, q_ok, col, D);
            gop[st] = row8(a.dO + head, qidx, q_ok, col, D);
            const bf16x8 o8 = row8(a.O + head, qidx, q_ok, col, D);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dpart = __builtin_fmaf((float)gop[st][e], (float)o8[e], dpart);
        }
        const float dsum = wave_half_sum(dpart);
        const float l2 = q_ok ? a.LSE[(size_t)bh * N + qidx] * kLog2e : 0.f;
        if (q_ok && half == 0) {
            a.L2[(size_t)bh * N + qidx] = l2;
            a.Dsum[(size_t)bh * N + qidx] = -dsum;  // negated: the dK/dV kernel's dP starts from it
        }

        f32x16 dq[S::kDBlocks];
#pragma unroll
        for (int b = 0; b < S::kDBlocks; ++b)
            dq[b] = f32x16{};

        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // One 64-key tile t in buffer set P = t % 2 (compile-time, so that the
        // buffer addresses fold into the LDS read offsets).  MASKED tiles may
        // hold keys after some query of the workgroup; the others need no mask.
        auto tile = [&](int t, auto parity_tag, auto masked_tag) __attribute__((always_inline)) {
            constexpr int P = decltype(parity_tag)::value;
            constexpr bool MASKED = decltype(masked_tag)::value;
            char *kc = P ? sk1 : sk0, *vc = P ? sv1 : sv0;
            off.opaque();
            if (t + 1 < t_end) {  // the other buffers were released by the last barrier
                load_tile<D>(Kh, kv_end, (t + 1) * kTile, P ? sk0 : sk1, wave_u, off.dma);
                load_tile<D>(Vh, kv_end, (t + 1) * kTile, P ? sv0 : sv1, wave_u, off.dma);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int key0 = t * kTile + kb * kRows;
                // Nothing to do for a wave past N, or (causal) a block whose
                // every key comes after every query of the wave.
                if (!wave_live || (CAUSAL && key0 > qw0 + kRows - 1))
                    continue;
                const char *kbase = kc + kb * kRows * S::kRowBytes;
                const char *vbase = vc + kb * kRows * S::kRowBytes;
                const f32x16 s = rows_times<D>(kbase, off, qop);
                const f32x16 dp = rows_times<D>(vbase, off, gop);
                // Register 4 j + e holds key key0 + 8 j + 4 half + e.  Keys past
                // N have zero K and V rows: their dS multiplies a zero K row.
                const bool masked = CAUSAL && MASKED && key0 + kRows - 1 > qw0;
                // Key key0 + 8 (r >> 2) + 4 half + (r & 3) is masked iff
                // 8 (r >> 2) + (r & 3) > thr.
                const int thr = masked ? qidx - key0 - 4 * half : kRows;
                float p[16], ds[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c_log2, -l2));
                    p[r] = (8 * (r >> 2) + (r & 3) > thr) ? 0.f : p[r];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    ds[r] = p[r] * (dp[r] - dsum);
                bf16x8 dsb[2];
                pack_b(ds, dsb);
                tr_times<D>(dq, kbase, off, dsb);
                // The exps need only S: they run under the dP products.  Operand
                // reads stay about two products ahead.
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int i = 0; i < S::kSteps; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // S
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
#pragma unroll
                for (int i = 0; i < S::kSteps; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // dP
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        // Causal: key tiles before q0 are visible to every query of the
        // workgroup (q0 is a multiple of two tiles, so they come in pairs).
        const int t_free = CAUSAL ? q0 / kTile : 0;
        int t = 0;
        for (; t < t_free; t += 2) {
            tile(t, std::integral_constant<int, 0>{}, std::false_type{});
            tile(t + 1, std::integral_constant<int, 1>{}, std::false_type{});
        }
        for (; t < t_end; t += 2) {
            tile(t, std::integral_constant<int, 0>{}, std::true_type{});
            if (t + 1 < t_end)
                tile(t + 1, std::integral_constant<int, 1>{}, std::true_type{});
        }
        if (q_ok)
            store_rows<D>(a.dQ + head + (size_t)qidx * D, dq, a.scale, half);
    }
#endif
}

// ---------------------------------------------------------------------------
// dK and dV: one workgroup per key block of one head.  Per 32-query block:
// S = Q K^T and dP = dO V^T (queries x keys), P = exp2(S c_log2 - L2),
// dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(Shape<D>::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dkdv_kernel(
    const BArgs a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using S = Shape<D>;
    __shared__ __attribute__((aligned(1024))) char sq0[S::kBytes];
    __shared__ __attribute__((aligned(1024))) char sq1[S::kBytes];
    __shared__ __attribute__((aligned(1024))) char sg0[S::kBytes];
    __shared__ __attribute__((aligned(1024))) char sg1[S::kBytes];
    __shared__ __attribute__((aligned(256))) float sl0[kTile], sl1[kTile], sd0[kTile], sd1[kTile];

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave_u = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int n = lane & 31, half = lane >> 5;
    const int N = a.N, nblk = a.ntiles;

    int bh, unit, npass;
    block_of(a, nblk, CAUSAL, bh, unit, npass);
    const size_t head = (size_t)bh * (size_t)N * D;
    const __bf16 *Qh = a.Q + head, *Gh = a.dO + head;
    const float *L2h = a.L2 + (size_t)bh * N, *Dh = a.Dsum + (size_t)bh * N;

    for (int pass = 0; pass < npass; ++pass) {
        // Per-lane LDS offsets, built afresh in each pass from an opaque copy of
        // the lane index so that they are not held live across passes.
        int lane_p = lane;
        asm volatile("" : "+v"(lane_p));
        Offsets<D> off(wave_u, lane_p);
        // One query tile (Q, dO, L2, D) into buffer set `second`.
        auto load_all = [&](int t, bool second) __attribute__((always_inline)) {
            load_tile<D>(Qh, N, t * kTile, second ? sq1 : sq0, wave_u, off.dma);
            load_tile<D>(Gh, N, t * kTile, second ? sg1 : sg0, wave_u, off.dma);
            if (wave_u == 0)
                load_vec(L2h, N, t * kTile, second ? sl1 : sl0, lane);
            else if (wave_u == 1)
                load_vec(Dh, N, t * kTile, second ? sd1 : sd0, lane);
        };
        if (pass > 0)
            __syncthreads();
        // (longest first: the heaviest key block is the first, which every
        // query sees)
        const int k0 = (CAUSAL && a.lpt ? unit : pair_block(CAUSAL, nblk, unit, pass)) * S::kBlock;
        const int kw0 = k0 + wave_u * kRows;
        const int kidx = kw0 + n;
        const bool k_ok = kidx < N;
        const bool wave_live = kw0 < N;
        // Causal: queries before k0 see none of the block's keys.
        const int t_lo = CAUSAL ? k0 / kTile : 0;
        const int t_end = (N + kTile - 1) / kTile;

        load_all(t_lo, false);

        // K^T and V^T operands, resident: k-step st holds columns
        // 16 st + 8 half .. +7 of this lane's key row.
        bf16x8 kop[S::kSteps], vop[S::kSteps];
#pragma unroll
        for (int st = 0; st < S::kSteps; ++st) {
            const int col = 16 * st + 8 * half;
            kop[st] = row8(a.K + head, kidx, k_ok, col, D);
            vop[st] = row8(a.V + head, kidx, k_ok, col, D);
        }
        f32x16 dk[S::kDBlocks], dv[S::kDBlocks];
#pragma unroll
        for (int b = 0; b < S::kDBlocks; ++b) {
            dk[b] = f32x16{};
            dv[b] = f32x16{};
        }

        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // One 64-query tile t in buffer set P = (t - t_lo) % 2 (compile-time, so
        // that the buffer addresses fold into the LDS read offsets).
        auto tile = [&](int t, auto parity_tag) __attribute__((always_inline)) {
            constexpr bool second = decltype(parity_tag)::value != 0;
            const char *qc = second ? sq1 : sq0, *gc = second ? sg1 : sg0;
            const float *lc = second ? sl1 : sl0, *dc = second ? sd1 : sd0;
            off.opaque();
            if (t + 1 < t_end)
                load_all(t + 1, !second);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int qs0 = t * kTile + qb * kRows;
                // Nothing to do for a wave past N, or (causal) a block whose
                // every query comes before every key of the wave.
                if (!wave_live || (CAUSAL && qs0 + kRows - 1 < kw0))
                    continue;
                const char *qbase = qc + qb * kRows * S::kRowBytes;
                const char *gbase = gc + qb * kRows * S::kRowBytes;
                // Register 4 j + e holds query qs0 + 8 j + 4 half + e.  The dP
                // product starts from -D of those queries (the workspace holds
                // -D), so it yields dP - D with no VALU subtraction.  Queries
                // past N have zero Q and dO rows and L2 = D = 0: p = 1 there,
                // but both products it feeds multiply a zero row.
                f32x16 neg_d;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 d4 = *LDS_PTR(const f32x4, dc + qb * kRows + 8 * j + 4 * half);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        neg_d[4 * j + e] = d4[e];
                }
                const f32x16 s = rows_times<D>(qbase, off, kop);
                const f32x16 dpd = rows_times<D>(gbase, off, vop, neg_d);
                const bool masked = CAUSAL && qs0 < kw0 + kRows - 1;
                // Query qs0 + 8 j + 4 half + e is masked iff 8 j + e < thr.
                const int thr = masked ? kidx - qs0 - 4 * half : 0;
                float p[16], ds[16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int qr = qb * kRows + 8 * j + 4 * half;
                    const f32x4 l4 = *LDS_PTR(const f32x4, lc + qr);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * j + e;
                        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c_log2, -l4[e]));
                        pr = (8 * j + e < thr) ? 0.f : pr;
                        p[r] = pr;
                        ds[r] = pr * dpd[r];
                    }
                }
                bf16x8 pb[2], dsb[2];
                pack_b(p, pb);
                pack_b(ds, dsb);
                tr_times<D>(dv, gbase, off, pb);
                tr_times<D>(dk, qbase, off, dsb);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        for (int t = t_lo; t < t_end; t += 2) {
            tile(t, std::integral_constant<int, 0>{});
            if (t + 1 < t_end)
                tile(t + 1, std::integral_constant<int, 1>{});
        }
        if (k_ok) {
            store_rows<D>(a.dK + head + (size_t)kidx * D, dk, a.scale, half);
            store_rows<D>(a.dV + head + (size_t)kidx * D, dv, 1.f, half);
        }
    }
#endif
}

template <int D, bool CAUSAL>
static hipError_t launch(const AttnBwdLaunch &l)
{
    BArgs a;
    a.Q = (const __bf16 *)l.q;
    a.K = (const __bf16 *)l.k;
    a.V = (const __bf16 *)l.v;
    a.O = (const __bf16 *)l.o;
    a.dO = (const __bf16 *)l.dout;
    a.LSE = l.lse;
    a.L2 = (float *)l.workspace;
    a.Dsum = (float *)l.workspace + (size_t)l.BH * l.N;
    a.dQ = (__bf16 *)l.dq;
    a.dK = (__bf16 *)l.dk;
    a.dV = (__bf16 *)l.dv;
    a.BH = (int)l.BH;
    a.N = (int)l.N;
    using S = Shape<D>;
    a.ntiles = (int)((l.N + S::kBlock - 1) / S::kBlock);
    // Causal: pairs of blocks, or single blocks longest first when the pairs
    // would not fill the chip's workgroup slots twice (256 CUs, 8 / kWaves
    // workgroups each) and the heads split evenly over the XCDs.
    const int64_t pairs = l.BH * ((a.ntiles + 1) / 2);
    a.lpt = CAUSAL && l.BH % kXcds == 0 && pairs < 2 * 256 * (8 / S::kWaves);
    a.n_wg = (int)(l.BH * ((CAUSAL && !a.lpt) ? (a.ntiles + 1) / 2 : a.ntiles));
    a.c_log2 = l.scale * kLog2e;
    a.scale = l.scale;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL>), dim3(a.n_wg), dim3(S::kThreads), 0, l.stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL>), dim3(a.n_wg), dim3(S::kThreads), 0, l.stream, a);
    return hipGetLastError();
}

}  // namespace bwd
}  // namespace attn_gfx950

int64_t attn_bwd_workgroups(int64_t BH, int64_t N)
{
    return BH * ((N + attn_gfx950::bwd::kBlockMin - 1) / attn_gfx950::bwd::kBlockMin);
}

hipError_t attn_bwd_launch(const AttnBwdLaunch &l)
{
    using namespace attn_gfx950::bwd;
    if (l.d == 128)
        return l.causal ? launch<128, true>(l) : launch<128, false>(l);
    return l.causal ? launch<64, true>(l) : launch<64, false>(l);
}
