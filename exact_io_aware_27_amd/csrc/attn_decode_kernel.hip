// attn_decode_kernel.hip -- key ranges of exact attention for a few query
// rows (decoding), streamed from HBM into registers.
//
// With one to four query rows per head, the forward kernel's 32-row MFMA
// tiles are almost empty and its LDS staging bounds the bytes in flight; the
// work is reading K and V once, and the HBM reads are what it costs (the
// IO-awareness principle of "FlashAttention evolution", letsgetai.github.io,
// FlashAttention (2022) section), so this kernel is built around the stream.
// It computes, per key range, the same partial result as the forward
// kernel's split mode (normalised O in fp32 and the range's LSE; the
// two-block merge equation of the "FlashAttention evolution" core-mechanism
// section combines the ranges afterwards).
//
// gfx950 mapping
//   * One 4-wave workgroup per (batch*head, key range); each wave streams a
//     contiguous quarter of the range through its own buffer resource, so
//     loads past the wave's keys read zeros with no memory access.
//   * d / 8 lanes hold one key row (16 bytes each), so one buffer_load_dwordx4
//     by the wave covers 64 / (d / 8) consecutive keys (1 KB contiguous); the
//     lanes of one row form a group, and group g takes keys g, g + G, ... of
//     the wave's run (G groups).
//   * The stream is double-buffered in registers: while one half (kHalf
//     slots of K and V) is consumed, the other half's loads are in flight,
//     8 KB of K and 8 KB of V per wave.  (A rotating ring of single slots
//     lost its wait counts at the loop head: the compiler then waited for
//     every load.)
//   * q.k: four v_dot2_f32_bf16 per lane, then a DPP butterfly over the
//     row's lanes.  Each group keeps its own exact online softmax per query
//     row (running max m, sum l, O over its 8 columns); groups merge by
//     permlane swaps, waves through LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn_gfx950 {
namespace decode {

constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
[[maybe_unused]] constexpr int kHalf = 8;  // slots per half of the double-buffered stream

template <int D>
struct Geo {
    static constexpr int kLanesPerRow = D / 8;              // 16 bytes of a row per lane
    static constexpr int kGroups = kWave / kLanesPerRow;    // keys per wave-wide load
    static constexpr int kRowBytes = D * 2;
};

// v_permlane16_swap_b32 a, b: lanes 16..31 and 48..63 of a trade places
// with lanes 0..15 and 32..47 of b.  From a = b = x, a then holds the even
// 16-lane rows of x twice and b the odd ones, so op(a, b) combines row r
// with row r ^ 1 in every lane.  Inline asm for the reason given at
// half_swap; the s_nops cover the VALU-write to permlane-read hazard.
__device__ __forceinline__ void row_swap(float &a, float &b)
{
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// Sum over the lanes of one key row, by DPP inside each 16-lane row.
//   d = 128 (16 lanes a key): row_ror 8, row_ror 4, then quad_perm swaps of
//   2 and 1 lanes.
//   d = 64 (8 lanes a key): row_half_mirror (lane i with lane 7 - i of its
//   8), then the same two quad_perm swaps; no step crosses an 8-lane half.
template <int D>
__device__ __forceinline__ float row_sum(float x)
{
    auto dpp = [](float v, auto ctrl_tag) {
        constexpr int C = decltype(ctrl_tag)::value;
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), C, 0xf, 0xf, false));
    };
    if constexpr (D == 128) {
        x += dpp(x, std::integral_constant<int, 0x128>{});  // row_ror 8
        x += dpp(x, std::integral_constant<int, 0x124>{});  // row_ror 4
    } else {
        x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
    }
    x += dpp(x, std::integral_constant<int, 0x4E>{});  // quad_perm [2, 3, 0, 1]
    x += dpp(x, std::integral_constant<int, 0xB1>{});  // quad_perm [1, 0, 3, 2]
    return x;
}

// Online-softmax state of one query row over the keys a group has seen
// (log2 units): running max m, sum l, and this lane's 8 columns of the
// unnormalised O.
struct State {
    float m, l;
    float o[8];
};

// Merge state b into a (the two-block merge equation).
__device__ __forceinline__ void merge(State &a, const State &b)
{
    const float m = fmaxf(a.m, b.m);
    const float fa = a.m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(a.m - m);
    const float fb = b.m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(b.m - m);
    a.m = m;
    a.l = a.l * fa + b.l * fb;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        a.o[j] = a.o[j] * fa + b.o[j] * fb;
}

struct DArgs {
    const __bf16 *Q, *K, *V;
    float *Opart, *LSEpart;  // [splits][BH][Nq][D], [splits][BH][Nq]
    int BH, Nq, Nk, n_splits, split_keys;
    float c_log2;
};

template <int D, bool CAUSAL, int NQ>
__global__ __launch_bounds__(kThreads) void attn_decode_kernel(const DArgs a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using G = Geo<D>;
    __shared__ float s_m[kWaves][NQ], s_l[kWaves][NQ];
    __shared__ __attribute__((aligned(16))) float s_o[kWaves][NQ][D];

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane / G::kLanesPerRow;         // key group of this lane
    const int c = lane % G::kLanesPerRow;         // 16-byte column chunk of the row
    const int bh = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
    const int Nq = a.Nq, Nk = a.Nk;

    // This wave's keys: a quarter of the range (split_keys is a multiple of
    // 128, so each quarter is whole 32-key blocks).
    const int kv_lo = split * a.split_keys;
    const int kv_hi = min(Nk, kv_lo + a.split_keys);
    const int wkeys = a.split_keys / kWaves;
    const int w_lo = min(kv_hi, kv_lo + wave * wkeys);
    const int w_hi = min(kv_hi, w_lo + wkeys);
    const int nkeys = w_hi - w_lo;
    const size_t row0 = (size_t)bh * Nk + w_lo;
    // Buffer resources over exactly this wave's rows: a load past them reads
    // zeros and touches no memory.
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.K + row0 * D), (short)0, (int)((uint32_t)nkeys * (uint32_t)G::kRowBytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.V + row0 * D), (short)0, (int)((uint32_t)nkeys * (uint32_t)G::kRowBytes), kBufferFlags);
    // Lane l loads chunk c of key g of each wave-wide slot of G keys.
    const uint32_t lane_off = (uint32_t)(g * G::kRowBytes + 16 * c);
    constexpr uint32_t kSlotBytes = G::kGroups * G::kRowBytes;  // 1 KB

    // Query rows: this lane's 8 columns of each.
    bf16x8 q[NQ];
    int lim[NQ];  // keys of this wave's run visible to query i: run index < lim
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int qi = min(i, Nq - 1);
        q[i] = *reinterpret_cast<const bf16x8 *>(a.Q + ((size_t)bh * Nq + qi) * D + 8 * c);
        // causal: query qi sees keys <= qi + Nk - Nq
        lim[i] = CAUSAL ? min(nkeys, qi + Nk - Nq + 1 - w_lo) : nkeys;
    }

    State st[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        st[i].m = kNegInf;
        st[i].l = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            st[i].o[j] = 0.f;
    }

    // One key (this lane's chunk of its K and V rows, run index key) into
    // every query's state.  The bf16 pairs are taken by shufflevector:
    // bit-casting the words of a packed vector indexed in an unrolled loop
    // gets all four dot products fed its first word by the compiler.
    auto consume = [&](const u32x4 &kraw, const u32x4 &vraw, int key) __attribute__((always_inline)) {
        const bf16x8 kw = __builtin_bit_cast(bf16x8, kraw);
        const bf16x8 vw = __builtin_bit_cast(bf16x8, vraw);
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = (float)vw[j];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            float s = 0.f;
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q[i], q[i], 0, 1),
                                                __builtin_shufflevector(kw, kw, 0, 1), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q[i], q[i], 2, 3),
                                                __builtin_shufflevector(kw, kw, 2, 3), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q[i], q[i], 4, 5),
                                                __builtin_shufflevector(kw, kw, 4, 5), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q[i], q[i], 6, 7),
                                                __builtin_shufflevector(kw, kw, 6, 7), s, false);
            s = row_sum<D>(s);
            const float x = key < lim[i] ? s * a.c_log2 : kNegInf;
            const float m = fmaxf(st[i].m, x);
            // both terms are 0 * (O, l) and a 0 weight while nothing is visible
            const float alpha = st[i].m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(st[i].m - m);
            const float p = x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x - m);
            st[i].m = m;
            st[i].l = __builtin_fmaf(st[i].l, alpha, p);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                st[i].o[j] = __builtin_fmaf(st[i].o[j], alpha, p * v[j]);
        }
    };

    // The stream: slot t holds keys G t .. G t + G - 1 of the run.  Halves A
    // and B of kHalf slots alternate: B's loads fly while A is consumed,
    // then A's next loads while B is.
    const int nslots = (nkeys + G::kGroups - 1) / G::kGroups;
    u32x4 ka[kHalf], va[kHalf], kb[kHalf], vb[kHalf];
    auto load = [&](u32x4 *kd, u32x4 *vd, int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < kHalf; ++r) {
            const int soff = (int)((uint32_t)(t0 + r) * kSlotBytes);
            kd[r] = __builtin_amdgcn_raw_buffer_load_b128(krs, lane_off, soff, 0);
            vd[r] = __builtin_amdgcn_raw_buffer_load_b128(vrs, lane_off, soff, 0);
        }
    };
    auto eat = [&](const u32x4 *kd, const u32x4 *vd, int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < kHalf; ++r)
            consume(kd[r], vd[r], G::kGroups * (t0 + r) + g);
    };
    // (The scheduling barriers keep each half's loads issued together ahead
    // of the other half's work; left free, the scheduler sinks them next to
    // their uses to save registers, and nothing is in flight.)
    load(ka, va, 0);
    for (int t0 = 0; t0 < nslots; t0 += 2 * kHalf) {
        load(kb, vb, t0 + kHalf);
        __builtin_amdgcn_sched_barrier(0);
        eat(ka, va, t0);
        __builtin_amdgcn_sched_barrier(0);
        load(ka, va, t0 + 2 * kHalf);
        __builtin_amdgcn_sched_barrier(0);
        eat(kb, vb, t0 + kHalf);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Merge the groups of the wave: rows of 16 lanes (permlane16 / 32
    // swaps), and at d = 64 the two 8-lane groups of each row first.
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        auto combine = [&](auto swap) __attribute__((always_inline)) {
            State b;
            float ma = st[i].m, mb = st[i].m;
            swap(ma, mb);
            float la = st[i].l, lb = st[i].l;
            swap(la, lb);
            State aa;
            aa.m = ma;
            aa.l = la;
            b.m = mb;
            b.l = lb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float oa = st[i].o[j], ob = st[i].o[j];
                swap(oa, ob);
                aa.o[j] = oa;
                b.o[j] = ob;
            }
            merge(aa, b);
            st[i] = aa;
        };
        if constexpr (D == 64)
            combine([](float &x, float &y) __attribute__((always_inline)) {
                // lanes 8..15 of each row trade with lanes 0..7 (row_ror 8)
                y = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xf, 0xf,
                                                                       false));
            });
        combine([](float &x, float &y) __attribute__((always_inline)) { row_swap(x, y); });
        combine([](float &x, float &y) __attribute__((always_inline)) { half_swap(x, y); });
    }

    // Across the waves through LDS; the first wave writes the range's result.
    if (lane < G::kLanesPerRow) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            if (lane == 0) {
                s_m[wave][i] = st[i].m;
                s_l[wave][i] = st[i].l;
            }
            *reinterpret_cast<f32x4 *>(&s_o[wave][i][8 * c]) = f32x4{st[i].o[0], st[i].o[1], st[i].o[2], st[i].o[3]};
            *reinterpret_cast<f32x4 *>(&s_o[wave][i][8 * c + 4]) =
                f32x4{st[i].o[4], st[i].o[5], st[i].o[6], st[i].o[7]};
        }
    }
    __syncthreads();
    if (wave == 0 && lane < G::kLanesPerRow) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            if (i >= Nq)
                break;
            State tot;
            tot.m = s_m[0][i];
            tot.l = s_l[0][i];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                tot.o[j] = s_o[0][i][8 * c + j];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                State b;
                b.m = s_m[w][i];
                b.l = s_l[w][i];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    b.o[j] = s_o[w][i][8 * c + j];
                merge(tot, b);
            }
            const size_t r = ((size_t)split * a.BH + bh) * Nq + i;
            const float inv = tot.l > 0.f ? 1.f / tot.l : 0.f;
            float *op = a.Opart + r * D + 8 * c;
            *reinterpret_cast<f32x4 *>(op) = f32x4{tot.o[0] * inv, tot.o[1] * inv, tot.o[2] * inv, tot.o[3] * inv};
            *reinterpret_cast<f32x4 *>(op + 4) =
                f32x4{tot.o[4] * inv, tot.o[5] * inv, tot.o[6] * inv, tot.o[7] * inv};
            if (c == 0)  // natural log, as the merge reads it
                a.LSEpart[r] = tot.l > 0.f ? (tot.m + __builtin_log2f(tot.l)) * 0.69314718055994530942f : kNegInf;
        }
    }
#endif
}

template <int D, bool CAUSAL, int NQ>
static hipError_t launch(const AttnLaunch &l, int splits, int split_keys)
{
    DArgs a;
    a.Q = (const __bf16 *)l.q;
    a.K = (const __bf16 *)l.k;
    a.V = (const __bf16 *)l.v;
    a.Opart = (float *)l.workspace;
    a.LSEpart = (float *)l.workspace + (size_t)splits * l.BH * l.Nq * D;
    a.BH = (int)l.BH;
    a.Nq = (int)l.Nq;
    a.Nk = (int)l.Nk;
    a.n_splits = splits;
    a.split_keys = split_keys;
    a.c_log2 = l.scale * kLog2e;
    hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, NQ>), dim3((unsigned)(l.BH * splits)), dim3(kThreads), 0,
                       l.stream, a);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_nq(const AttnLaunch &l, int splits, int split_keys)
{
    switch (l.Nq) {
    case 1:
        return launch<D, CAUSAL, 1>(l, splits, split_keys);
    case 2:
        return launch<D, CAUSAL, 2>(l, splits, split_keys);
    case 3:
        return launch<D, CAUSAL, 3>(l, splits, split_keys);
    default:
        return launch<D, CAUSAL, 4>(l, splits, split_keys);
    }
}

}  // namespace decode
}  // namespace attn_gfx950

hipError_t attn_decode_ranges_launch(const AttnLaunch &l, int splits, int split_keys)
{
    using namespace attn_gfx950::decode;
    if (l.d == 128)
        return l.causal ? launch_nq<128, true>(l, splits, split_keys) : launch_nq<128, false>(l, splits, split_keys);
    return l.causal ? launch_nq<64, true>(l, splits, split_keys) : launch_nq<64, false>(l, splits, split_keys);
}
