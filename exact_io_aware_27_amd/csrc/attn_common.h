// attn_common.h -- vector types and wave-level helpers shared by the gfx950
// attention kernels (forward and backward).  Device code only; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_gfx950 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.44269504088896340736f;
// Buffer-resource word 3 for raw (unformatted, stride-0) 32-bit loads with
// out-of-range offsets returning zero.
constexpr int kBufferFlags = 0x00020000;

// v_permlane32_swap_b32 a, b exchanges lanes 32..63 of a with lanes 0..31 of
// b.  Starting from a = b = x this leaves a = [x_lo, x_lo], b = [x_hi, x_hi],
// so op(a, b) combines lane l with lane l^32 in every lane.  It is issued as
// inline asm with two read-write operands: the compiler builtin's second
// result gets dropped when both operands carry the same value.  The asm is
// not volatile, so the scheduler may move it like any VALU instruction; the
// s_nops cover the VALU-write to permlane-read hazard the compiler cannot see
// inside the asm.
__device__ __forceinline__ void half_swap(float &a, float &b)
{
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
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

// Position pos of `count` dispatch positions of one XCD -> the work rank it
// takes.  The XCD deals its positions to its 32 CUs in rounds of 32; odd
// rounds run backwards (the last round over its own length), so a CU that
// takes a heavy rank in one round takes a light one in the next.  A
// permutation of [0, count).
constexpr int kCusPerXcd = 32;  // MI355X: 256 CUs over 8 XCDs
__device__ __forceinline__ int snake_slot(int pos, int count)
{
    const int round = pos / kCusPerXcd, i = pos % kCusPerXcd;
    const int len = min(kCusPerXcd, count - round * kCusPerXcd);
    return (round & 1) ? round * kCusPerXcd + (len - 1 - i) : pos;
}

// Logical workgroup order: XCD-major (consecutive logical indices share an
// XCD, so the units of one head stay on one XCD), then head-major.
__device__ __forceinline__ void unit_of(int wg, int n_wg, int n_units, int &bh, int &unit)
{
    const int xcd = wg % kXcds;
    const int slot = wg / kXcds;
    const int per = n_wg / kXcds;
    const int extra = n_wg % kXcds;
    const int lin = xcd * per + (xcd < extra ? xcd : extra) + slot;
    bh = lin / n_units;
    unit = lin % n_units;
}

}  // namespace attn_gfx950
