// attn_fp8_kernel.hip -- FP8 attention forward for gfx950: block quantization
// with incoherent processing, then the fused attention on FP8 operands.
//
// The FP8 mode of FlashAttention-3 as the pages outline it: both products on
// FP8 matrix cores, one scale per block of the inputs instead of one per
// tensor, and Q and K multiplied by a random orthogonal matrix before they are
// quantized so that outliers spread over the head dimension ("FlashAttention
// evolution", letsgetai.github.io, FlashAttention-3 section; "FlashAttention
// 1-4 evolution cheat sheet", argus-lessons, FlashAttention-3 section).
//
// Formats (head dim 128):
//   * FP8 is OCP E4M3, round to nearest even.
//   * A quantization block is 64 rows of one head.  Its scale is 2^E with E
//     the smallest integer such that the block's largest magnitude is at most
//     448 * 2^E, stored as the E8M0 byte E + 127.  Power-of-two scales are
//     what the gfx950 scaled MFMA applies itself
//     (v_mfma_scale_f32_32x32x64_f8f6f4), so dequantization costs nothing.
//   * Incoherent processing: x -> (x * s) H, random signs s, then the
//     Sylvester Hadamard matrix H by its fast transform in fp32 (butterfly
//     stages of stride 1, 2, ..., 64, each (a, b) -> (a + b, a - b)).  The
//     product of rotated Q and K is d times the original.
//   * Q alone is then multiplied in fp32 by c = scale * log2(e) (and 1/d when
//     rotated) before it is quantized, so that Q K^T comes out of the matrix
//     cores as the logits in log2 units: the attention kernel applies no
//     scale, and it starts every score product from the negated reference
//     max in the accumulator, so that p = exp2 of the product's result.
//   * Q and K: [BH][Np][128] bytes, Np = N rounded up to 64, rows past N zero.
//     V: transposed, [BH][128][Np], and within every 64-key tile the keys are
//     stored in the order the P operand of the P V product holds them: key r
//     at position 32 ((r >> 2) & 1) + 16 (r >> 5) + 4 ((r >> 3) & 3) + (r & 3).
//   * Exponents: one E8M0 byte per block, [BH][Np / 64].
//
// The attention kernel is the bf16 forward's design at FP8 rates: a
// workgroup of 8 waves owns 256 queries (32 per wave) and walks 128-key tiles
// (two 64-key blocks), double-buffered in LDS through buffer_load ... lds, one
// barrier per tile; per 64-key block each wave computes S^T = K Q^T (two
// 32-key halves, two K = 64 MFMAs each), the softmax against a lagging
// reference max, and O^T += V^T P^T (four MFMAs over the block's 64 keys).
// The softmax of block s runs while the matrix cores compute S of block s+1
// (minus the reference, taken in the accumulator) and P V of block s-1; K
// and V are copied two blocks ahead of their use.  P is rounded to E4M3
// for the product (the reference may lag the row max by at most 8 in log2
// units, so P <= 256 stays inside E4M3); O is divided by the fp32 sum of the
// unrounded P, which also gives the LSE.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn_gfx950 {
namespace fp8 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kRowsBlk = 64;                 // quantization block = K/V tile rows
constexpr int kWaves = 8;
constexpr int kThreads = kWave * kWaves;
constexpr int kBr = 32 * kWaves;             // queries per workgroup
[[maybe_unused]] constexpr int kTileBytes = 2 * kRowsBlk * kD;  // one K or V^T tile (128 keys): 16 KB
[[maybe_unused]] constexpr float kRefSlack = 8.f;  // P <= 2^8 inside E4M3's 448
constexpr int kE8M0One = 127;

// ---------------------------------------------------------------------------
// Quantization

// Smallest E with amax <= 448 * 2^E, from the bits of amax = (1 + f) 2^e:
// E = e - 8 when 1 + f <= 1.75, else e - 7; 0 for amax == 0; E8M0 range.
__device__ __forceinline__ int block_exp(float amax)
{
    if (!(amax > 0.f))
        return 0;
    const uint32_t u = __float_as_uint(amax);
    const int e = (int)((u >> 23) & 0xffu) - 127;
    const int E = (u & 0x7fffffu) <= 0x600000u ? e - 8 : e - 7;
    return max(-127, min(127, E));
}

// DPP moves within rows of 16 lanes (no LDS traffic): quad_perm, and
// row_ror n, where lane i reads lane (i - n) mod 16 of its row.  BANKS
// selects the groups of 4 lanes written; mov leaves the others undefined,
// update keeps them from `old`.
template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, BANKS, false));
}

template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_update(float old, float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, x), CTRL, 0xf, BANKS, false));
}

// One butterfly stage across the 16 lanes of a row: lane c pairs with lane
// c ^ m; the lower lane of a pair keeps a + b, the upper one a - b (a the
// lower lane's value).  fma(+-1, v, o) rounds exactly as v + o and o - v.
template <int M>
__device__ __forceinline__ float row_butterfly(float v, float sign)
{
    float o;
    if constexpr (M == 1)
        o = dpp_mov<0xB1, 0xf>(v);  // quad_perm [1, 0, 3, 2]
    else if constexpr (M == 2)
        o = dpp_mov<0x4E, 0xf>(v);  // quad_perm [2, 3, 0, 1]
    else if constexpr (M == 8)
        o = dpp_mov<0x128, 0xf>(v);  // row_ror 8
    else {  // M == 4: lanes 0-3 and 8-11 read 4 ahead, lanes 4-7 and 12-15 4 behind
        o = dpp_mov<0x12C, 0x5>(v);        // row_ror 12 (lane i reads i - 12 = i + 4) into banks 0, 2
        o = dpp_update<0x124, 0xa>(o, v);  // row_ror 4 (lane i reads i - 4) into banks 1, 3
    }
    return __builtin_fmaf(sign, v, o);
}

// One 64-row block of one head per workgroup (256 threads); thread t owns
// columns 8 (t % 16) .. +7 of four rows: rows 16 p + t / 16 (p = 0..3), or,
// for the transposed V, the consecutive rows 4 (t / 16) + p.  ROTATE applies
// the signs and the fast Hadamard transform (three stages inside a thread,
// four across the 16 lanes of a row, through DPP moves); SCALE then
// multiplies every value by `mul` in fp32 (Q's softmax scale in log2 units);
// TRANSPOSE converts
// column by column (the four rows of one column are four consecutive bytes of
// the tile's key order) and writes V^T through LDS.
template <bool ROTATE, bool TRANSPOSE, bool SCALE>
__global__ __launch_bounds__(256) void quantize_kernel(const __bf16 *__restrict__ x, uint8_t *__restrict__ out,
                                                       uint8_t *__restrict__ exps, int N, int Np, int nblk,
                                                       uint32_t s0, uint32_t s1, uint32_t s2, uint32_t s3, float mul)
{
    __shared__ float wmax[4];
    // V^T staging: column c's 64 key bytes at 64 c, 16-byte chunk q of it at
    // chunk q ^ ((c >> 3) & 3), which spreads a column-wise write over banks.
    __shared__ __attribute__((aligned(16))) uint8_t tr[TRANSPOSE ? kD * kRowsBlk : 16];
    const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
    const int t = threadIdx.x, c16 = t & 15, rsub = t >> 4;
    auto row_of = [&](int p) { return TRANSPOSE ? 4 * rsub + p : 16 * p + rsub; };
    float sgn[4];  // +1 for the lower lane of a stage-m pair, -1 for the upper
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sgn[i] = (c16 >> i) & 1 ? -1.f : 1.f;
    float v[4][8];
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = blk * kRowsBlk + row_of(p);
        bf16x8 in = bf16x8{};
        if (row < N)
            in = *reinterpret_cast<const bf16x8 *>(x + ((size_t)bh * N + row) * kD + 8 * c16);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[p][e] = (float)in[e];
        if constexpr (ROTATE) {
            const uint32_t sw = (c16 < 4) ? s0 : (c16 < 8) ? s1 : (c16 < 12) ? s2 : s3;
            const uint32_t bits = sw >> (8 * (c16 & 3));  // columns 8 c16 .. +7
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if ((bits >> e) & 1u)
                    v[p][e] = -v[p][e];
#pragma unroll
            for (int h = 1; h < 8; h *= 2)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if ((i & h) == 0) {
                        const float a = v[p][i], b = v[p][i + h];
                        v[p][i] = a + b;
                        v[p][i + h] = a - b;
                    }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[p][e] = row_butterfly<1>(v[p][e], sgn[0]);
                v[p][e] = row_butterfly<2>(v[p][e], sgn[1]);
                v[p][e] = row_butterfly<4>(v[p][e], sgn[2]);
                v[p][e] = row_butterfly<8>(v[p][e], sgn[3]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (SCALE)
                v[p][e] *= mul;
            amax = fmaxf(amax, fabsf(v[p][e]));
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m *= 2)
        amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    if ((t & 63) == 0)
        wmax[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const int E = block_exp(amax);
    auto fp8x4 = [&](float a, float b, float c, float d) {  // E4M3 bytes of (a, b, c, d) / 2^E, a lowest
        int u = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(a, -E), __builtin_amdgcn_ldexpf(b, -E), 0,
                                                false);
        u = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(c, -E), __builtin_amdgcn_ldexpf(d, -E), u, true);
        return (uint32_t)u;
    };
    if constexpr (!TRANSPOSE) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x2 w = {fp8x4(v[p][0], v[p][1], v[p][2], v[p][3]), fp8x4(v[p][4], v[p][5], v[p][6], v[p][7])};
            *reinterpret_cast<u32x2 *>(out + ((size_t)bh * Np + blk * kRowsBlk + row_of(p)) * kD + 8 * c16) = w;
        }
    } else {
        // rows 4 rsub + p sit at key positions base + p
        const int base = 32 * (rsub & 1) + 16 * (rsub >> 3) + 4 * ((rsub >> 1) & 3);
        const int chunk = base >> 4, within = base & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int col = 8 * c16 + e;
            *reinterpret_cast<uint32_t *>(tr + col * kRowsBlk + 16 * (chunk ^ (c16 & 3)) + within) =
                fp8x4(v[0][e], v[1][e], v[2][e], v[3][e]);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ch = t + 256 * i, col = ch >> 2, part = ch & 3;
            *reinterpret_cast<u32x4 *>(out + ((size_t)bh * kD + col) * Np + blk * kRowsBlk + 16 * part) =
                *reinterpret_cast<const u32x4 *>(tr + col * kRowsBlk + 16 * (part ^ ((col >> 3) & 3)));
        }
    }
    if (t == 0)
        exps[(size_t)bh * nblk + blk] = (uint8_t)(E + kE8M0One);
}

// ---------------------------------------------------------------------------
// Attention

// LDS swizzle (16-byte chunk c of row r at chunk position c ^ swz(r)).  K
// rows and V^T rows of a 128-key tile are both 128 bytes, two per 256-byte
// bank line; a ds_read_b128 by lanes 0..15 reads rows 0..15 at one chunk:
// distinct positions need (r & 1, c ^ swz(r)) distinct, which
// (r & 7) ^ ((r >> 3) & 1) gives.
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct F8Args {
    const uint8_t *Q, *K, *VT;       // [BH][Np][128], [BH][Np][128], [BH][128][Np]
    const uint8_t *qe, *ke, *ve;     // [BH][Np / 64] E8M0
    __bf16 *O;                        // [BH][N][128]
    float *LSE;                       // [BH][N] or null
    int BH, N, Np, nblk, n_wg, nqt;
};

__device__ __forceinline__ f32x16 mfma8(const i32x8 &a, const i32x8 &b, const f32x16 &c, int sa, int sb)
{
    // cbsz = blgp = 0: both operands E4M3; the E8M0 scales multiply A and B.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ i32x8 lds_pair(const char *p0, const char *p1)
{
    const i32x4 lo = *LDS_PTR(const i32x4, p0);
    const i32x4 hi = *LDS_PTR(const i32x4, p1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_fp8_kernel(
    const F8Args a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __shared__ __attribute__((aligned(1024))) char sk0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sk1[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sv0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sv1[kTileBytes];
    // Each thread's pending rescale factor (set when its row's reference
    // moves, applied to O after the next P V): only the rare paths touch it,
    // so it waits here rather than in a register.
    __shared__ float s_alpha[kThreads];

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave_u = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int N = a.N, Np = a.Np, nqt = a.nqt;

    const int n_units = CAUSAL ? (nqt + 1) / 2 : nqt;
    int bh, unit;
    unit_of(blockIdx.x, a.n_wg, n_units, bh, unit);
    const int npass = (CAUSAL && nqt - 1 - unit != unit) ? 2 : 1;

    const uint8_t *Kh = a.K + (size_t)bh * Np * kD;
    const uint8_t *Vh = a.VT + (size_t)bh * kD * Np;
    const __amdgpu_buffer_rsrc_t vrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)Vh, (short)0, (int)((uint32_t)kD * (uint32_t)Np), kBufferFlags);

    for (int pass = 0; pass < npass; ++pass) {
        const int qt = CAUSAL ? (pass == 0 ? nqt - 1 - unit : unit) : unit;
        if (pass > 0)
            __syncthreads();
        // Per-lane offsets, computed afresh in each pass from an opaque copy of
        // the lane index so that they are not kept live across passes.  A tile
        // holds 128 keys (two 64-key blocks): K as 128 rows of 128 bytes, V^T
        // as 128 rows (head dim) of 128 bytes (keys).  DMA: wave w copies 1 KB
        // slices 2 w and 2 w + 1 of each, rows 8 s + lane / 8, chunk lane % 8.
        int lane_p = lane;
        asm volatile("" : "+v"(lane_p));
        const int n = lane_p & 31, half = lane_p >> 5;
        uint32_t kdma[2], vdma[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 8 * (2 * wave_u + i) + lane_p / 8, pos = lane_p % 8;
            kdma[i] = (uint32_t)(r * kD + ((pos ^ swz_k(r)) << 4));
            vdma[i] = (uint32_t)(r * Np + ((pos ^ swz_k(r)) << 4));
        }
        // S operand: row n of a 32-key block, bytes 64 st + 32 half .. +31
        // (chunks 4 st + 2 half + c).  P V operand of block b64 of a tile: V^T
        // row n of a 32-row block, bytes 64 b64 + 32 half .. +31 (chunks
        // 4 b64 + 2 half + c).  Both swizzles repeat every 16 rows, so the
        // two operands share one set of offsets (koff[b64][c] for V^T).
        uint32_t koff[2][2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                koff[st][c] = (uint32_t)(n * kD + (((4 * st + 2 * half + c) ^ swz_k(n)) << 4));
        const int q0 = qt * kBr;
        const int qw0 = q0 + 32 * wave_u;
        const int qidx = qw0 + n;
        const bool q_ok = qidx < N;
        const int kv_end = CAUSAL ? min(N, q0 + kBr) : N;
        const int nb_end = (kv_end + kRowsBlk - 1) / kRowsBlk;  // 64-key blocks
        const int t_end = (nb_end + 1) / 2;                      // 128-key tiles
        const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)Kh, (short)0, (int)((uint32_t)kv_end * (uint32_t)kD), kBufferFlags);

        // Tile t of K (rows past kv_end: zeros, no memory access) and of V^T
        // (keys 128 t .. +127 of every row; keys past the row belong to no
        // visible block and are never multiplied by a nonzero P).
        auto load_k = [&](int t, char *buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, LDS_PTR(void, buf + (2 * wave_u + i) * 1024), 16,
                                                         kdma[i], (int)((uint32_t)t * (uint32_t)kTileBytes), 0, 0);
        };
        auto load_v = [&](int t, char *buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, LDS_PTR(void, buf + (2 * wave_u + i) * 1024), 16,
                                                         vdma[i], (int)((uint32_t)t * (uint32_t)(2 * kRowsBlk)), 0, 0);
        };
        // Block exponents by scalar loads of the dword holding the byte (a
        // dword-aligned read holding an in-range byte stays inside one page);
        // scalar loads are counted apart from the tile copies, so waiting for
        // one never waits for the other.
        auto exp_of = [&](const uint8_t *base, int blk) __attribute__((always_inline)) {
            const size_t g = (size_t)bh * a.nblk + (size_t)min(blk, a.nblk - 1);
            const uint32_t word = ((const __attribute__((address_space(4))) uint32_t *)base)[g >> 2];
            return (int)((word >> (8 * (g & 3))) & 0xffu);
        };

        load_k(0, sk0);
        load_k(1, sk1);
        load_v(0, sv0);
        // V buffer 1 is multiplied by the zero P of "block -1" in the first
        // step: it must hold finite values.
#pragma unroll
        for (int i = 0; i < kTileBytes / (16 * kThreads); ++i)
            *LDS_PTR(u32x4, sv1 + 16 * (tid + i * kThreads)) = u32x4{};

        // Q^T operand (E4M3 bytes 64 st + 32 half .. +31 of this lane's query
        // row) and its block exponent, shared by the wave (32 queries of one
        // 64-row block).
        i32x8 qop[2];
        {
            const uint8_t *qrow = a.Q + ((size_t)bh * Np + (q_ok ? qidx : 0)) * kD + 32 * half;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const i32x4 lo = *reinterpret_cast<const i32x4 *>(qrow + 64 * st);
                const i32x4 hi = *reinterpret_cast<const i32x4 *>(qrow + 64 * st + 16);
                qop[st] = q_ok ? i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]} : i32x8{};
            }
        }
        const int qs = qw0 < N ? (int)a.qe[(size_t)bh * a.nblk + qw0 / kRowsBlk] : kE8M0One;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        // Scores of 64-key block b64 of the tile in K buffer kbuf, in log2
        // units (Q was quantized with the softmax scale and log2 e folded in),
        // added to `init`: the reference max is subtracted in the matrix
        // product's accumulator, so p = exp2 of the result with no VALU work.
        auto scores = [&](const char *kbuf, int b64, int ks, f32x16 *s, const f32x16 &init)
            __attribute__((always_inline)) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                s[b] = init;
#pragma unroll
                for (int st = 0; st < 2; ++st)
                    s[b] = mfma8(lds_pair(kbuf + (64 * b64 + 32 * b) * kD + koff[st][0],
                                          kbuf + (64 * b64 + 32 * b) * kD + koff[st][1]),
                                 qop[st], s[b], ks, qs);
            }
        };
        f32x16 sc[2];
        scores(sk0, 0, exp_of(a.ke, 0), sc, f32x16{});

        // Register 4 j + e of 32-key half b holds key 64 s + 32 b + 8 j + 4 half + e
        // of 64-key block s.
        auto visible = [&](int blk, int b, int r) __attribute__((always_inline)) {
            const int key = 64 * blk + 32 * b + 8 * (r >> 2) + 4 * half + (r & 3);
            return key < N && (!CAUSAL || key <= qidx);
        };
        // The reference max m (log2 units) lives in neg_m, which holds -m in
        // every register (0 while the row has seen no key, m = -inf): the
        // accumulator every score product starts from, so scores arrive
        // relative to the reference.  A row whose next block passes m_thr
        // (kRefSlack; -inf while no key was seen) moves the reference.
        float m_thr;
        f32x16 neg_m;
        auto set_ref = [&](float m) __attribute__((always_inline)) {
            m_thr = (m == kNegInf) ? kNegInf : kRefSlack;
            const float m_sub = (m == kNegInf) ? 0.f : m;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                neg_m[r] = -m_sub;
        };
        auto ref_sub = [&]() __attribute__((always_inline)) { return -neg_m[0]; };
        auto ref_max = [&]() __attribute__((always_inline)) { return m_thr == kNegInf ? kNegInf : -neg_m[0]; };
        {
            float mx = kNegInf;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, visible(0, b, r) ? sc[b][r] : kNegInf);
            set_ref(wave_half_max(mx));
            // the first block's scores were formed before the reference existed
#pragma unroll
            for (int b = 0; b < 2; ++b)
                sc[b] += neg_m;
        }
        f32x16 oacc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            oacc[b] = f32x16{};
        float l_run = 0.f;
        bool pending = false;
        // This thread's slot of s_alpha, its lane index computed afresh where
        // it is used (from an opaque all-ones mask, so that it is neither
        // hoisted nor kept live through the key loop for the rare paths).
        auto alpha_slot = [&]() __attribute__((always_inline)) -> float & {
            uint32_t all = ~0u;
            asm volatile("" : "+s"(all));
            const int l = (int)__builtin_amdgcn_mbcnt_hi(all, __builtin_amdgcn_mbcnt_lo(all, 0u));
            return s_alpha[wave_u * kWave + l];
        };
        i32x8 pb_prev = i32x8{};
        // Block exponents, loaded one step ahead of their use, so that no
        // scalar load's latency sits in front of a step's first MFMA (the
        // steps' rare branches keep the compiler from hoisting them): ks_next
        // is that of the K block whose scores the next step forms, vs_next
        // that of the V block whose P V it accumulates.
        int ks_next = exp_of(a.ke, 1), vs_next = kE8M0One;

        // One 64-key step: block s = 2 t + J of tile t (K buffer P = t % 2).
        // The softmax of block s interleaves with the scores of block s+1 and
        // P V of block s-1:
        //   J = 0: scores of block 2t+1 (tile t, K buffer P, rows 64..127),
        //          P V of block 2t-1 (tile t-1, V buffer 1-P, keys 64..127);
        //   J = 1: scores of block 2t+2 (tile t+1, K buffer 1-P, rows 0..63),
        //          P V of block 2t (tile t, V buffer P, keys 0..63), and the
        //          copies of K tile t+2 into K buffer P and V tile t+1 into V
        //          buffer 1-P (both released before the tile's barrier).
        // MASKED: block s needs the causal / sequence-end mask; NEXT_MASKED:
        // block s+1 does (past the last block every key is invisible).
        auto step = [&](int t, auto parity_tag, auto half_tag, auto masked_tag, auto next_masked_tag)
            __attribute__((always_inline)) {
            constexpr int P = decltype(parity_tag)::value;
            constexpr int J = decltype(half_tag)::value;
            constexpr bool MASKED = decltype(masked_tag)::value;
            constexpr bool NEXT_MASKED = decltype(next_masked_tag)::value;
            char *kown = P ? sk1 : sk0, *kother = P ? sk0 : sk1;
            char *vown = P ? sv1 : sv0, *vother = P ? sv0 : sv1;
            const char *knext = J == 0 ? kown : kother;
            const char *vprev = J == 0 ? vother : vown;
            constexpr int knext_b64 = J == 0 ? 1 : 0, vprev_b64 = J == 0 ? 1 : 0;
            const int blk = 2 * t + J;
            if constexpr (J == 1) {
                load_k(t + 2, kown);
                load_v(t + 1, vother);
            }
            const int ks = ks_next, vs = vs_next;
            ks_next = exp_of(a.ke, blk + 2);
            vs_next = exp_of(a.ve, blk);
            // Keep the LDS offsets opaque (so they ride in the ds_read offset
            // field instead of being hoisted as per-buffer sums) and the
            // softmax inside its step.
#pragma unroll
            for (int st = 0; st < 2; ++st)
                asm volatile("" : "+v"(koff[st][0]), "+v"(koff[st][1]));
            asm volatile("" : "+v"(sc[0]), "+v"(sc[1]));

            // P of block s against the reference, rounded to E4M3 in the order
            // of the P V operand: byte 4 w + i is register 4 (w & 3) + i of
            // 32-key half w >> 2.
            float p[2][16];
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    p[b][r] = __builtin_amdgcn_exp2f(sc[b][r]);
                    if constexpr (MASKED)
                        p[b][r] = visible(blk, b, r) ? p[b][r] : 0.f;
                }
            float rs0 = p[0][0], rs1 = p[0][1];
#pragma unroll
            for (int r = 2; r < 32; r += 2) {
                rs0 += p[r >> 4][r & 15];
                rs1 += p[r >> 4][(r & 15) + 1];
            }
            l_run += rs0 + rs1;
            i32x8 pb;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const float *pp = &p[w >> 2][4 * (w & 3)];
                // Low half, then high half into the same register.  As asm, the
                // first conversion needs no register cleared before it (the
                // builtin's "old" operand is a zero the compiler materialises
                // with a v_mov, 8 per step, though the high half is written
                // next).
                int u;
                asm("v_cvt_pk_fp8_f32 %0, %1, %2" : "=v"(u) : "v"(pp[0]), "v"(pp[1]));
                asm("v_cvt_pk_fp8_f32 %0, %1, %2 op_sel:[0,0,1]" : "+v"(u) : "v"(pp[2]), "v"(pp[3]));
                pb[w] = u;
            }

            f32x16 sn[2];
            scores(knext, knext_b64, ks, sn, neg_m);
#pragma unroll
            for (int db = 0; db < 4; ++db)
                oacc[db] = mfma8(lds_pair(vprev + db * 32 * kD + koff[vprev_b64][0],
                                          vprev + db * 32 * kD + koff[vprev_b64][1]),
                                 pb_prev, oacc[db], vs, kE8M0One);

            float mx;
            if constexpr (NEXT_MASKED) {
                mx = kNegInf;
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        mx = fmaxf(mx, visible(blk + 1, b, r) ? sn[b][r] : kNegInf);
            } else {  // every key visible
                float m0 = sn[0][0];
#pragma unroll
                for (int r = 1; r < 32; ++r)
                    m0 = fmaxf(m0, sn[r >> 4][r & 15]);
                mx = m0;
            }
            const bool reref = __builtin_amdgcn_ballot_w64(mx > m_thr) != 0;

            // The step's region: 8 MFMAs, each followed by the operand reads
            // for the MFMAs after it and a share of the softmax VALU work.
            // (Not in the masked steps without the causal mask, which only
            // the ragged end of a sequence runs: left to the default
            // scheduler, they fit the register budget.)
            if constexpr (CAUSAL || !MASKED) {
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // reads before the VALU share: 1.8% faster
                    __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);   // exp
                    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // other VALU
                }
            }
            asm volatile("" : "+v"(pb), "+v"(l_run));

            // Both branches are rare: laid out off the step's straight line,
            // so that a step runs into the next without a taken branch.
            if (__builtin_expect(pending, 0)) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    oacc[b] *= alpha_slot();
            }
            pending = reref;
            if (__builtin_expect(reref, 0)) {
                const float m_old = ref_sub(), m_ref = ref_max();
                const float m_new = fmaxf(m_ref, wave_half_max(mx + m_old));
                const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                alpha_slot() = alpha;
                l_run *= alpha;
                set_ref(m_new);
                // the next block's scores were formed against the old reference
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    sn[b] -= (ref_sub() - m_old);
            }
            sc[0] = sn[0];
            sc[1] = sn[1];
            pb_prev = pb;
        };
        // One 128-key tile: block 2t, the barrier (K tile t+1 and V tile t have
        // landed; every wave is done with K tile t and V tile t-1), block 2t+1.
        auto tile = [&](int t, auto parity_tag, auto masked_tag, auto mid_masked_tag, auto next_masked_tag)
            __attribute__((always_inline)) {
            step(t, parity_tag, std::integral_constant<int, 0>{}, masked_tag, mid_masked_tag);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            step(t, parity_tag, std::integral_constant<int, 1>{}, mid_masked_tag, next_masked_tag);
        };
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using Unmasked = std::false_type;
        using Masked = std::true_type;
        // Blocks [0, b_free) need no mask: inside the sequence and at or below
        // the causal diagonal of every query of the workgroup.  Whole unmasked
        // tile pairs run in the first loop; the last one is peeled because the
        // block after it needs the mask.
        int b_free = N / kRowsBlk;
        if (CAUSAL)
            b_free = min(b_free, (q0 + 1) / kRowsBlk);
        b_free = min(b_free, nb_end);
        const int t_free = (b_free / 2) & ~1;  // unmasked tiles, an even count
        int t = 0;
        for (; t + 2 < t_free; t += 2) {
            tile(t, P0{}, Unmasked{}, Unmasked{}, Unmasked{});
            tile(t + 1, P1{}, Unmasked{}, Unmasked{}, Unmasked{});
        }
        if (t < t_free) {
            tile(t, P0{}, Unmasked{}, Unmasked{}, Unmasked{});
            tile(t + 1, P1{}, Unmasked{}, Unmasked{}, Masked{});
            t += 2;
        }
        for (; t < t_end; t += 2) {
            tile(t, P0{}, Masked{}, Masked{}, Masked{});
            if (t + 1 < t_end)
                tile(t + 1, P1{}, Masked{}, Masked{}, Masked{});
        }
        // P V of the last block, 2 t_end - 1 (second half of the last tile,
        // whose V landed at that tile's barrier); then drain the copies still
        // in flight before the next pass reuses the buffers.
        {
            char *vlast = ((t_end - 1) & 1) ? sv1 : sv0;
            const int vs = vs_next;
#pragma unroll
            for (int db = 0; db < 4; ++db)
                oacc[db] = mfma8(lds_pair(vlast + db * 32 * kD + koff[1][0], vlast + db * 32 * kD + koff[1][1]),
                                 pb_prev, oacc[db], vs, kE8M0One);
            if (__builtin_expect(pending, 0)) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    oacc[b] *= alpha_slot();
            }
            // O is read only by the lanes of valid queries: keep these MFMAs
            // out of that lane-masked branch (an MFMA under a partial EXEC mask
            // does not compute the lanes' tile).
            asm volatile("" : "+v"(oacc[0]), "+v"(oacc[1]), "+v"(oacc[2]), "+v"(oacc[3]));
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        const float l_tot = wave_half_sum(l_run);
        if (q_ok) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            __bf16 *orow = a.O + ((size_t)bh * N + qidx) * kD;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    u32x2 w;
                    w[0] = pack_bf16x2(oacc[b][4 * j + 0] * inv, oacc[b][4 * j + 1] * inv);
                    w[1] = pack_bf16x2(oacc[b][4 * j + 2] * inv, oacc[b][4 * j + 3] * inv);
                    *reinterpret_cast<u32x2 *>(orow + 32 * b + 8 * j + 4 * half) = w;
                }
            if (a.LSE != nullptr && half == 0)
                a.LSE[(size_t)bh * N + qidx] = (ref_max() + __builtin_log2f(l_tot)) * 0.69314718055994530942f;
        }
    }
#endif
}

}  // namespace fp8
}  // namespace attn_gfx950

int64_t attn_fp8_rows(int64_t N) { return (N + 63) / 64 * 64; }

hipError_t attn_fp8_quantize_launch(const AttnFp8Quantize &q)
{
    using namespace attn_gfx950::fp8;
    const int Np = (int)attn_fp8_rows(q.N), nblk = Np / kRowsBlk;
    const int grid = (int)(q.BH * nblk);
    const uint32_t *s = q.sign_bits;
    const uint32_t s0 = s ? s[0] : 0, s1 = s ? s[1] : 0, s2 = s ? s[2] : 0, s3 = s ? s[3] : 0;
    const __bf16 *x = (const __bf16 *)q.x;
    uint8_t *out = (uint8_t *)q.out, *exps = (uint8_t *)q.exps;
    // (a multiplier of exactly 1 is skipped: the product would change nothing)
    const bool scale = q.mul != 1.f;
    if (q.transpose)
        hipLaunchKernelGGL((quantize_kernel<false, true, false>), dim3(grid), dim3(256), 0, q.stream, x, out, exps,
                           (int)q.N, Np, nblk, 0u, 0u, 0u, 0u, 1.f);
    else if (s && scale)
        hipLaunchKernelGGL((quantize_kernel<true, false, true>), dim3(grid), dim3(256), 0, q.stream, x, out, exps,
                           (int)q.N, Np, nblk, s0, s1, s2, s3, q.mul);
    else if (s)
        hipLaunchKernelGGL((quantize_kernel<true, false, false>), dim3(grid), dim3(256), 0, q.stream, x, out, exps,
                           (int)q.N, Np, nblk, s0, s1, s2, s3, 1.f);
    else if (scale)
        hipLaunchKernelGGL((quantize_kernel<false, false, true>), dim3(grid), dim3(256), 0, q.stream, x, out, exps,
                           (int)q.N, Np, nblk, 0u, 0u, 0u, 0u, q.mul);
    else
        hipLaunchKernelGGL((quantize_kernel<false, false, false>), dim3(grid), dim3(256), 0, q.stream, x, out, exps,
                           (int)q.N, Np, nblk, 0u, 0u, 0u, 0u, 1.f);
    return hipGetLastError();
}

hipError_t attn_fp8_launch(const AttnFp8Launch &l)
{
    using namespace attn_gfx950::fp8;
    F8Args a;
    a.Q = (const uint8_t *)l.q8;
    a.K = (const uint8_t *)l.k8;
    a.VT = (const uint8_t *)l.vt8;
    a.qe = (const uint8_t *)l.qe;
    a.ke = (const uint8_t *)l.ke;
    a.ve = (const uint8_t *)l.ve;
    a.O = (__bf16 *)l.o;
    a.LSE = l.lse;
    a.BH = (int)l.BH;
    a.N = (int)l.N;
    a.Np = (int)attn_fp8_rows(l.N);
    a.nblk = a.Np / kRowsBlk;
    a.nqt = (int)((l.N + kBr - 1) / kBr);
    a.n_wg = (int)(l.BH * (l.causal ? (a.nqt + 1) / 2 : a.nqt));
    if (l.causal)
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<true>), dim3(a.n_wg), dim3(kThreads), 0, l.stream, a);
    else
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<false>), dim3(a.n_wg), dim3(kThreads), 0, l.stream, a);
    return hipGetLastError();
}
