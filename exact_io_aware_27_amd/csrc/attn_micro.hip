// attn_micro.hip -- microbenchmarks of the gfx950 issue rates that the
// attention kernels' design rests on (libattn_micro.so; not part of the
// attention ABI in include/attn.h).
//
// The FlashAttention-4 section of "FlashAttention 1-4 evolution cheat sheet"
// (argus-lessons) prices one forward tile by counting cycles per unit: matrix
// work, exponentials, shared-memory reads.  These kernels measure the gfx950
// numbers for the same count, in shader-clock cycles read from the wave's own
// counter (s_memtime), so the results do not depend on the clock the chip
// runs at; the clock itself is measured beside them (s_memtime cycles against
// the constant-rate s_memrealtime counter).
//
//   rate:  one kind of VALU instruction on 16 independent chains per lane (or
//          one dependent chain), w waves per SIMD: cycles per instruction per
//          SIMD (throughput) or per dependent instruction (latency).
//   mix:   32x32x16 bf16 MFMAs on four independent accumulators, each
//          followed by k FMAs and e exponentials (v_exp_f32, or exp2_poly)
//          on independent chains, interleaved by sched_group_barrier as the
//          attention kernel interleaves its step: cycles per MFMA per SIMD.
//   lds:   LDS read throughput (ds_read_b128, ds_read_b64_tr_b16): bytes
//          per cycle per CU.
//   mix_lds: MFMAs whose streamed operand is read from LDS in the step's
//          issue order, with no VALU: cycles per MFMA per SIMD.
//   hbm:   a plain read stream over a large buffer: GB/s, the ceiling of a
//          bandwidth-bound kernel's reads.
//
// Occupancy is pinned: one workgroup per CU (96 KB of LDS each) of 4 w waves,
// so every SIMD holds exactly w waves.  256 workgroups fill the 256 CUs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_common.h"
#include "exp2_poly.h"

namespace attn_gfx950 {
namespace micro {

constexpr int kLdsBytes = 96 * 1024;  // > 160 KB / 2: one workgroup per CU
constexpr int kChains = 16;

enum Op { kOpFma = 0, kOpExp = 1, kOpPoly = 2, kOpMul = 3 };

template <int OP>
__device__ __forceinline__ float apply(float x)
{
    if constexpr (OP == kOpFma)
        return __builtin_fmaf(x, 0.999f, 0.001f);
    else if constexpr (OP == kOpExp)
        return __builtin_amdgcn_exp2f(-x);  // neg is an input modifier: one instruction
    else if constexpr (OP == kOpPoly)
        return exp2_poly(-x);
    else
        return x * 0.999f;
}

// Each wave stores its own start and end stamps (shader cycles and real-time
// ticks); the host takes a workgroup's span as the latest end minus the
// earliest start, since the waves sharing a SIMD need not finish together.
__device__ __forceinline__ void record(unsigned long long *times, uint64_t c0, uint64_t r0)
{
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        const size_t i = ((size_t)blockIdx.x * (blockDim.x / kWave) + wave) * 4;
        times[i] = c0;
        times[i + 1] = c1;
        times[i + 2] = r0;
        times[i + 3] = r1;
    }
}

// DEP = false: 16 independent chains, 16 instructions per iteration.
// DEP = true: one chain, 16 dependent instructions per iteration.
template <int OP, bool DEP>
__global__ __launch_bounds__(1024) void rate_kernel(float *sink, unsigned long long *times, int iters)
{
    extern __shared__ char lds_pin[];
    float x[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        x[i] = 0.25f + 0.001f * (float)((threadIdx.x + i) & 63);
    if (threadIdx.x == 0)
        lds_pin[0] = 0;
    __syncthreads();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        if constexpr (DEP) {
#pragma unroll
            for (int i = 0; i < kChains; ++i)
                x[0] = apply<OP>(x[0]);
        } else {
#pragma unroll
            for (int i = 0; i < kChains; ++i)
                x[i] = apply<OP>(x[i]);
        }
        asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                     "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]),
                     "+v"(x[14]), "+v"(x[15]));
    }
    record(times, c0, r0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        s += x[i];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s + (float)lds_pin[threadIdx.x & 7];
}

// Four MFMAs per iteration on independent accumulators (CHAIN: all four on
// one accumulator, each waiting for the last, as the score product's k-steps
// do); after each, K FMAs and E exponentials (POLY: exp2_poly) on the 16
// independent chains (PAIRED: each exponential takes the result of the FMA
// just before it, as p = exp2(s c - m) does).
template <int K, int E, bool POLY, bool CHAIN = false, bool PAIRED = false>
__global__ __launch_bounds__(1024) void mix_kernel(float *sink, unsigned long long *times, int iters)
{
    extern __shared__ char lds_pin[];
    const int t = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)((t + i) & 63));
        b[i] = (__bf16)(0.002f * (float)((t + 3 * i) & 63));
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc[j] = f32x16{};
    float x[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        x[i] = 0.25f + 0.001f * (float)((t + i) & 63);
    if (t == 0)
        lds_pin[0] = 0;
    __syncthreads();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (CHAIN)
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[0], 0, 0, 0);
            else
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
            if constexpr (PAIRED) {
                // every chain takes one FMA per iteration; the last FMA of
                // each group is followed at once by an exponential of its
                // result, written back to the same chain
#pragma unroll
                for (int k = 0; k < K; ++k)
                    x[(j * K + k) % kChains] = apply<kOpFma>(x[(j * K + k) % kChains]);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    x[(j * K + K - 1 - e) % kChains] =
                        apply<POLY ? kOpPoly : kOpExp>(x[(j * K + K - 1 - e) % kChains]);
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k)
                    x[(j * (K + E) + k) % kChains] = apply<kOpFma>(x[(j * (K + E) + k) % kChains]);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    x[(j * (K + E) + K + e) % kChains] =
                        apply<POLY ? kOpPoly : kOpExp>(x[(j * (K + E) + K + e) % kChains]);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
            __builtin_amdgcn_sched_group_barrier(0x402, K + E * (POLY ? 9 : 1), 0);  // VALU incl. transcendental (exp2_poly of -x: 9)
        }
    }
    record(times, c0, r0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            s += acc[j][i];
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        s += x[i];
    sink[(size_t)blockIdx.x * blockDim.x + t] = s + (float)lds_pin[t & 7];
}

// LDS contents for the LDS kernels: small bf16 values (defined data, and
// MFMA inputs that toggle like real operands).
__device__ __forceinline__ void lds_fill(char *lds)
{
    for (int i = threadIdx.x; i < kLdsBytes / 16; i += blockDim.x) {
        const uint32_t w = 0x3c003c00u + ((uint32_t)(i * 2654435761u) & 0x00ff00ffu);
        *LDS_PTR(u32x4, lds + 16 * i) = u32x4{w, w ^ 0x00110011u, w ^ 0x00220022u, w ^ 0x00330033u};
    }
}

// One wave-wide LDS read of an MFMA A operand (8 bf16 a lane, 1 KB a wave):
// KIND 0 one ds_read_b128 (the K operand of the score product), KIND 1 two
// ds_read_b64_tr_b16 (the V^T operand of P V).  Lanes read consecutive
// addresses: no bank conflicts.
template <int KIND>
__device__ __forceinline__ bf16x8 lds_operand(const char *lds, uint32_t off, int j)
{
    const int lane = threadIdx.x & (kWave - 1);
    if constexpr (KIND == 0) {
        return *LDS_PTR(const bf16x8, lds + off + 16 * lane + 1024 * j);
    } else {
        const u32x2 lo = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, lds + off + 8 * lane + 1024 * j)));
        const u32x2 hi = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, lds + off + 8 * lane + 1024 * j + 512)));
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        return __builtin_bit_cast(bf16x8, w);
    }
}

// LDS read throughput: each wave issues 16 independent reads per iteration
// (KIND 0: ds_read_b128, 16 bytes a lane; KIND 1: ds_read_b64_tr_b16, 8
// bytes a lane) and waits for them; w waves per SIMD overlap their batches.
// Addresses stay below 16.5 KB of the 96 KB allocation.
template <int KIND>
__global__ __launch_bounds__(1024) void lds_rate_kernel(float *sink, unsigned long long *times, int iters)
{
    extern __shared__ char lds[];
    lds_fill(lds);
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t off = 0;
    uint32_t acc = 0;
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        asm volatile("" : "+v"(off));  // a fresh address each iteration: no read is hoisted
        if constexpr (KIND == 0) {
            u32x4 x[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                x[j] = *LDS_PTR(const u32x4, lds + off + 16 * lane + 1024 * j);
            asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]),
                         "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]),
                         "v"(x[14]), "v"(x[15]));
            acc ^= x[0][0] ^ x[15][3];
        } else {
            s16x4 x[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                x[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, lds + off + 8 * lane + 512 * j));
            asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]),
                         "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]),
                         "v"(x[14]), "v"(x[15]));
            acc ^= (uint32_t)(uint16_t)(x[0][0] ^ x[15][3]);
        }
    }
    record(times, c0, r0);
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc & 0xff);
}

// The attention step's matrix-core and LDS work without its softmax: 16
// MFMAs per iteration on four accumulators, the A operand of each (1 KB a
// wave) read from LDS inside the iteration: KIND 0 one ds_read_b128 each,
// KIND 1 two ds_read_b64_tr_b16 each, KIND 2 the step's mix (ds_read_b128
// for the first 8 MFMAs, as the score product reads K; the transposing pair
// for the last 8, as P V reads V^T).  The issue order is the step's: 4 reads
// up front, then per MFMA the MFMA and up to 2 reads for the MFMAs ahead.
// One or two waves per SIMD (the attention kernels run two), with the
// register budget of two stated: without it the scheduler keeps source
// order, each read right before its MFMA, to protect an occupancy the launch
// never uses.
template <int KIND>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void mix_lds_kernel(
    float *sink, unsigned long long *times, int iters)
{
    extern __shared__ char lds[];
    const int t = threadIdx.x;
    lds_fill(lds);
    __syncthreads();
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        b[i] = (__bf16)(0.002f * (float)((t + 3 * i) & 63));
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc[j] = f32x16{};
    uint32_t off = 0;
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        asm volatile("" : "+v"(off));  // a fresh address each iteration: no read is hoisted
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bf16x8 a = (KIND == 0 || (KIND == 2 && i < 8)) ? lds_operand<0>(lds, off, i)
                                                                  : lds_operand<KIND == 0 ? 0 : 1>(lds, off, i);
            acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i & 3], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        }
    }
    record(times, c0, r0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            s += acc[j][i];
    sink[(size_t)blockIdx.x * blockDim.x + t] = s;
}

// HBM read stream: every thread reads 16-byte words of a large buffer in a
// grid-stride loop, four loads in flight per iteration, and folds them into
// one word (written once, so the loads are not removed).  The ceiling a
// bandwidth-bound kernel of this chip can reach on reads alone.
// BLOCKED: each workgroup streams its own contiguous slice of the buffer,
// 16 KB per iteration (as a K/V stream walks one head), instead of the
// grid-wide interleave.
template <bool BLOCKED>
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4 *__restrict__ src, size_t n16,
                                                       uint32_t *__restrict__ sink)
{
    size_t i, end, stride;
    if constexpr (BLOCKED) {
        const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
        i = (size_t)blockIdx.x * per + threadIdx.x;
        end = min(n16, (size_t)(blockIdx.x + 1) * per);
        stride = blockDim.x;
    } else {
        i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
        end = n16;
        stride = (size_t)gridDim.x * blockDim.x;
    }
    u32x4 acc = {};
    for (; i + 3 * stride < end; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < end; i += stride)
        acc ^= src[i];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <typename F>
static int run(F kernel, int waves_per_simd, int iters, double *cycles, double *clock_ghz, double *ms)
{
    if (waves_per_simd < 1 || waves_per_simd > 4 || iters < 1)
        return 2;
    const int grid = 256, block = 4 * waves_per_simd * kWave, waves = grid * block / kWave;
    float *sink = nullptr;
    unsigned long long *times = nullptr;
    if (hipMalloc(&sink, (size_t)grid * block * sizeof(float)) != hipSuccess)
        return 7;
    if (hipMalloc(&times, (size_t)waves * 4 * sizeof(unsigned long long)) != hipSuccess) {
        (void)hipFree(sink);
        return 7;
    }
    int rate_khz = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev);
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    int status = 0;
    for (int rep = 0; rep < 3 && status == 0; ++rep) {  // the last of three launches is kept
        (void)hipEventRecord(e0, nullptr);
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), kLdsBytes, nullptr, sink, times, iters);
        (void)hipEventRecord(e1, nullptr);
        if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess)
            status = 7;
    }
    if (status == 0) {
        float t = 0.f;
        (void)hipEventElapsedTime(&t, e0, e1);
        unsigned long long *h = new unsigned long long[(size_t)waves * 4];
        if (hipMemcpy(h, times, (size_t)waves * 4 * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
            status = 7;
        const int per = block / kWave;
        double c = 0.0, r = 0.0;
        for (int g = 0; g < grid; ++g) {  // span of each workgroup: earliest start to latest end
            unsigned long long c_lo = ~0ull, c_hi = 0, r_lo = ~0ull, r_hi = 0;
            for (int w = 0; w < per; ++w) {
                const unsigned long long *e = h + ((size_t)g * per + w) * 4;
                c_lo = e[0] < c_lo ? e[0] : c_lo;
                c_hi = e[1] > c_hi ? e[1] : c_hi;
                r_lo = e[2] < r_lo ? e[2] : r_lo;
                r_hi = e[3] > r_hi ? e[3] : r_hi;
            }
            c += (double)(c_hi - c_lo);
            r += (double)(r_hi - r_lo);
        }
        delete[] h;
        c /= grid;
        r /= grid;
        *cycles = c;  // mean over workgroups of the shader cycles one workgroup's timed loops span
        *clock_ghz = rate_khz > 0 && r > 0 ? c / (r / (rate_khz * 1e3)) / 1e9 : 0.0;
        *ms = t;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(sink);
    (void)hipFree(times);
    return status;
}

// Elementwise exp2_poly and v_exp_f32 of n inputs (accuracy tests).
__global__ __launch_bounds__(256) void exp2_eval_kernel(const float *x, float *poly, float *hw, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        poly[i] = exp2_poly(x[i]);
        hw[i] = __builtin_amdgcn_exp2f(x[i]);
    }
}

}  // namespace micro
}  // namespace attn_gfx950

using namespace attn_gfx950::micro;

// One rate measurement: op (0 fma, 1 v_exp_f32, 2 exp2_poly, 3 mul),
// dependent (0: 16 independent chains, 1: one chain), waves per SIMD 1..4.
// out[0] = cycles per instruction per SIMD (independent: the SIMD's
// throughput over all its waves) or per dependent instruction (latency);
// out[1] = shader clock in GHz; out[2] = launch time in ms.  Returns 0, 2
// for arguments outside the table, 7 for a HIP error.
extern "C" __attribute__((visibility("default"))) int attn_micro_rate(int op, int dependent, int waves_per_simd,
                                                                      int iters, double *out)
{
    double cyc = 0, ghz = 0, ms = 0;
    int st = 2;
#define ATTN_MICRO_RATE(O)                                                                                  \
    if (op == O)                                                                                            \
        st = dependent ? run(rate_kernel<O, true>, waves_per_simd, iters, &cyc, &ghz, &ms)                   \
                       : run(rate_kernel<O, false>, waves_per_simd, iters, &cyc, &ghz, &ms);
    ATTN_MICRO_RATE(kOpFma)
    ATTN_MICRO_RATE(kOpExp)
    ATTN_MICRO_RATE(kOpPoly)
    ATTN_MICRO_RATE(kOpMul)
#undef ATTN_MICRO_RATE
    if (st != 0)
        return st;
    const double insts = (double)iters * kChains;
    out[0] = dependent ? cyc / insts : cyc / (insts * waves_per_simd);
    out[1] = ghz;
    out[2] = ms;
    return 0;
}

extern "C" __attribute__((visibility("default"))) int attn_micro_mix_shape(int k_fma, int n_exp, int poly, int shape,
                                                                           int waves_per_simd, int iters,
                                                                           double *out);

// One mix measurement: after each 32x32x16 bf16 MFMA, k_fma FMAs and n_exp
// exponentials (poly: exp2_poly instead of v_exp_f32).  Instances:
// (k, e) in (0,0) (2,1) (3,1) (4,1) (5,1) (6,1) (4,2) (8,0), and poly with
// (3,1) (4,1); shape 1 runs (0,0) and (4,1) with the MFMAs on one dependent
// accumulator chain, shape 2 runs (4,1) with each exponential taking the
// FMA just before it.  out[0] = cycles per MFMA per SIMD (32 = the matrix core's
// own rate for this shape), out[1] = shader clock (GHz), out[2] = ms,
// out[3] = whole-chip bf16 TFLOP/s of the MFMAs.
extern "C" __attribute__((visibility("default"))) int attn_micro_mix(int k_fma, int n_exp, int poly,
                                                                     int waves_per_simd, int iters, double *out)
{
    return attn_micro_mix_shape(k_fma, n_exp, poly, 0, waves_per_simd, iters, out);
}

// attn_micro_mix with a dependence shape: 0 as attn_micro_mix, 1 the MFMAs
// on one accumulator chain, 2 each exponential taking the FMA before it.
extern "C" __attribute__((visibility("default"))) int attn_micro_mix_shape(int k_fma, int n_exp, int poly, int shape,
                                                                           int waves_per_simd, int iters,
                                                                           double *out)
{
    double cyc = 0, ghz = 0, ms = 0;
    int st = 2;
    if (shape == 1 && !poly && ((k_fma == 0 && n_exp == 0) || (k_fma == 4 && n_exp == 1))) {
        st = k_fma ? run(mix_kernel<4, 1, false, true, false>, waves_per_simd, iters, &cyc, &ghz, &ms)
                   : run(mix_kernel<0, 0, false, true, false>, waves_per_simd, iters, &cyc, &ghz, &ms);
    } else if (shape == 2 && !poly && k_fma == 4 && n_exp == 1) {
        st = run(mix_kernel<4, 1, false, false, true>, waves_per_simd, iters, &cyc, &ghz, &ms);
    } else if (shape != 0) {
        return 2;
    }
#define ATTN_MICRO_MIX(K, E, P)                                                                 \
    if (shape == 0 && k_fma == K && n_exp == E && (poly != 0) == P)                             \
        st = run(mix_kernel<K, E, P>, waves_per_simd, iters, &cyc, &ghz, &ms);
    ATTN_MICRO_MIX(0, 0, false)
    ATTN_MICRO_MIX(2, 1, false)
    ATTN_MICRO_MIX(3, 1, false)
    ATTN_MICRO_MIX(4, 1, false)
    ATTN_MICRO_MIX(5, 1, false)
    ATTN_MICRO_MIX(6, 1, false)
    ATTN_MICRO_MIX(4, 2, false)
    ATTN_MICRO_MIX(8, 0, false)
    ATTN_MICRO_MIX(3, 1, true)
    ATTN_MICRO_MIX(4, 1, true)
#undef ATTN_MICRO_MIX
    if (st != 0)
        return st;
    const double mfmas = (double)iters * 4;
    out[0] = cyc / (mfmas * waves_per_simd);
    out[1] = ghz;
    out[2] = ms;
    out[3] = 256.0 * 4 * waves_per_simd * mfmas * 32768.0 / (ms * 1e-3) / 1e12;
    return 0;
}

// LDS read throughput: kind 0 ds_read_b128, 1 ds_read_b64_tr_b16; waves per
// SIMD 1..4.  out[0] = bytes read per shader cycle per CU (all its waves),
// out[1] = shader clock (GHz), out[2] = ms.  Returns 0, 2 for arguments
// outside the table, 7 for a HIP error.
extern "C" __attribute__((visibility("default"))) int attn_micro_lds_rate(int kind, int waves_per_simd, int iters,
                                                                          double *out)
{
    double cyc = 0, ghz = 0, ms = 0;
    int st = 2;
    if (kind == 0)
        st = run(lds_rate_kernel<0>, waves_per_simd, iters, &cyc, &ghz, &ms);
    else if (kind == 1)
        st = run(lds_rate_kernel<1>, waves_per_simd, iters, &cyc, &ghz, &ms);
    if (st != 0)
        return st;
    const double bytes = (double)iters * 16 * (kind == 0 ? 1024 : 512) * 4 * waves_per_simd;
    out[0] = bytes / cyc;
    out[1] = ghz;
    out[2] = ms;
    return 0;
}

// MFMAs fed from LDS: each 32x32x16 bf16 MFMA's A operand (1 KB a wave)
// read from LDS (kind 0 ds_read_b128, 1 two ds_read_b64_tr_b16, 2 the two as
// the attention step mixes them); one or two waves per SIMD.  out as
// attn_micro_mix.
extern "C" __attribute__((visibility("default"))) int attn_micro_mix_lds(int kind, int waves_per_simd, int iters,
                                                                         double *out)
{
    double cyc = 0, ghz = 0, ms = 0;
    int st = 2;
    if (waves_per_simd > 2)
        return 2;
    if (kind == 0)
        st = run(mix_lds_kernel<0>, waves_per_simd, iters, &cyc, &ghz, &ms);
    else if (kind == 1)
        st = run(mix_lds_kernel<1>, waves_per_simd, iters, &cyc, &ghz, &ms);
    else if (kind == 2)
        st = run(mix_lds_kernel<2>, waves_per_simd, iters, &cyc, &ghz, &ms);
    if (st != 0)
        return st;
    const double mfmas = (double)iters * 16;
    out[0] = cyc / (mfmas * waves_per_simd);
    out[1] = ghz;
    out[2] = ms;
    out[3] = 256.0 * 4 * waves_per_simd * mfmas * 32768.0 / (ms * 1e-3) / 1e12;
    return 0;
}

// HBM read bandwidth: `mib` MiB (at least 64) read by hbm_read_kernel on
// `wgs` workgroups of 256 threads (256..65536), grid-interleaved or
// (blocked != 0) one contiguous slice per workgroup, the last of `reps`
// launches (1..100) timed with HIP events.  out[0] = GB/s, out[1] = ms.
// Returns 0, 2 for arguments outside those ranges, 7 for a HIP error
// (allocation included).
extern "C" __attribute__((visibility("default"))) int attn_micro_hbm_read(int mib, int wgs, int reps, int blocked,
                                                                          double *out)
{
    if (mib < 64 || wgs < 256 || wgs > 65536 || reps < 1 || reps > 100)
        return 2;
    const size_t bytes = (size_t)mib << 20;
    void *src = nullptr;
    uint32_t *sink = nullptr;
    if (hipMalloc(&src, bytes) != hipSuccess)
        return 7;
    if (hipMalloc(&sink, (size_t)wgs * 256 * sizeof(uint32_t)) != hipSuccess) {
        (void)hipFree(src);
        return 7;
    }
    int status = hipMemset(src, 0x5a, bytes) == hipSuccess ? 0 : 7;
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    float ms = 0.f;
    for (int r = 0; r < reps && status == 0; ++r) {
        (void)hipEventRecord(e0, nullptr);
        if (blocked)
            hipLaunchKernelGGL(hbm_read_kernel<true>, dim3(wgs), dim3(256), 0, nullptr,
                               (const attn_gfx950::u32x4 *)src, bytes / 16, sink);
        else
            hipLaunchKernelGGL(hbm_read_kernel<false>, dim3(wgs), dim3(256), 0, nullptr,
                               (const attn_gfx950::u32x4 *)src, bytes / 16, sink);
        (void)hipEventRecord(e1, nullptr);
        if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess)
            status = 7;
    }
    if (status == 0) {
        (void)hipEventElapsedTime(&ms, e0, e1);
        out[0] = (double)bytes / (ms * 1e-3) / 1e9;
        out[1] = ms;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(src);
    (void)hipFree(sink);
    return status;
}

// poly[i] = exp2_poly(x[i]) and hw[i] = v_exp_f32(x[i]) for i < n; x, poly
// and hw are device arrays of n floats.  One kernel on `stream` (a
// hipStream_t as void*).  Returns 0, 2 for n < 0 or a null pointer, 7 for a
// launch error.
extern "C" __attribute__((visibility("default"))) int attn_micro_exp2(const float *x, float *poly, float *hw, int n,
                                                                      void *stream)
{
    if (n < 0 || (n > 0 && (!x || !poly || !hw)))
        return 2;
    if (n == 0)
        return 0;
    hipLaunchKernelGGL(exp2_eval_kernel, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), x,
                       poly, hw, n);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}
