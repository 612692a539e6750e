// attn_api.hip -- the C ABI of libattn.so (declared in include/attn.h).
//
// Every argument is checked before the first HIP runtime call, so all error
// codes except ATTN_HIP are reachable on a machine without a GPU.

#include <cmath>
#include <cstdint>

#include "../../include/attn.h"
#include "attn_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

// a * b into *out; false if the product leaves [0, INT64_MAX].
bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    if (a < 0 || b < 0)
        return false;
    if (a != 0 && b > INT64_MAX / a)
        return false;
    *out = a * b;
    return true;
}

bool overlaps(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

}  // namespace

extern "C" const char *attn_status_string(int status)
{
    switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_NULL_PTR: return "ATTN_NULL_PTR";
    case ATTN_BAD_SHAPE: return "ATTN_BAD_SHAPE";
    case ATTN_UNSUPPORTED_D: return "ATTN_UNSUPPORTED_D";
    case ATTN_BAD_SCALE: return "ATTN_BAD_SCALE";
    case ATTN_MISALIGNED: return "ATTN_MISALIGNED";
    case ATTN_ALIAS: return "ATTN_ALIAS";
    case ATTN_HIP: return "ATTN_HIP";
    default: return "ATTN_UNKNOWN_STATUS";
    }
}

extern "C" int attn_last_hip_error(void) { return g_last_hip_error; }

extern "C" int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                        void *stream)
{
    // 1. Shapes: non-negative, byte sizes and index ranges representable.
    int64_t BH, rows, elems, bytes, lse_bytes;
    if (B < 0 || H < 0 || N < 0 || !mul_ok(B, H, &BH) || !mul_ok(BH, N, &rows))
        return ATTN_BAD_SHAPE;
    // 2. Head dimension.
    if (d != 64 && d != 128)
        return ATTN_UNSUPPORTED_D;
    if (!mul_ok(rows, d, &elems) || !mul_ok(elems, 2, &bytes) || !mul_ok(rows, 4, &lse_bytes))
        return ATTN_BAD_SHAPE;
    if (N * d >= (int64_t(1) << 31))  // in-head offsets are 32-bit in the kernel
        return ATTN_BAD_SHAPE;
    if (rows > 0 && attn_workgroups(BH, N) > INT32_MAX)
        return ATTN_BAD_SHAPE;
    // 3. Scale.
    if (!std::isfinite(scale))
        return ATTN_BAD_SCALE;
    // 4. Empty problem: nothing to read or write.
    if (rows == 0)
        return ATTN_OK;
    // 5. Pointers.
    if (!q || !k || !v || !o)
        return ATTN_NULL_PTR;
    // 6. Alignment: 16-byte vector loads and stores of bf16 rows; 4-byte LSE.
    const auto mis16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
    if (mis16(q) || mis16(k) || mis16(v) || mis16(o) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
        return ATTN_MISALIGNED;
    // 7. Outputs must not overlap inputs or each other (q, k, v may alias one another).
    if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes))
        return ATTN_ALIAS;
    if (lse && (overlaps(lse, lse_bytes, q, bytes) || overlaps(lse, lse_bytes, k, bytes) ||
                overlaps(lse, lse_bytes, v, bytes) || overlaps(lse, lse_bytes, o, bytes)))
        return ATTN_ALIAS;

    AttnLaunch a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.BH = BH;
    a.N = N;
    a.d = d;
    a.causal = causal != 0;
    a.scale = scale;
    a.stream = static_cast<hipStream_t>(stream);
    const hipError_t err = attn_launch(a);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return ATTN_HIP;
    }
    return ATTN_OK;
}
