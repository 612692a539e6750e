// attn_api.hip -- the C ABI of libattn.so (declared in include/attn.h).
//
// Every argument is checked before the first HIP runtime call, so all error
// codes except ATTN_HIP are reachable on a machine without a GPU.

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/attn.h"
#include "attn_common.h"
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
    case ATTN_BAD_WORKSPACE: return "ATTN_BAD_WORKSPACE";
    case ATTN_BAD_ARGUMENT: return "ATTN_BAD_ARGUMENT";
    case ATTN_SCRATCH_TOO_SMALL: return "ATTN_SCRATCH_TOO_SMALL";
    default: return "ATTN_UNKNOWN_STATUS";
    }
}

extern "C" int attn_last_hip_error(void) { return g_last_hip_error; }

namespace {

// The scratch of attn_fwd_splitkv_noalloc: one array per GPU the library
// runs on (each device holds its own copy at its own address), kept until the
// process ends.  Host code never uses the array's name as an address: the
// name is a host-side stand-in, and a kernel handed it would fault.  Each
// device's address is looked up once with hipGetSymbolAddress and kept in
// g_scratch.
constexpr int64_t kScratchBytes = int64_t(32) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of the current device's scratch array; looked up on the
// first call on each device (with that device current).
hipError_t scratch_address(void **out)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

// Shared validation and launch of attn_fwd, attn_fwd_splitkv and
// attn_fwd_splitkv_noalloc, in the documented order.  use_scratch: the
// workspace arguments are ignored and the per-range partials go to the
// library's scratch array.
int fwd_common(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H,
               int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, int64_t num_splits,
               void *workspace, int64_t workspace_bytes, void *stream, bool use_scratch = false)
{
    // 1. Shapes: non-negative, byte sizes and index ranges representable.
    int64_t BH, qrows, krows, qelems, kelems, qbytes, kbytes, lse_bytes;
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || num_splits < 1 || !mul_ok(B, H, &BH) ||
        !mul_ok(BH, Nq, &qrows) || !mul_ok(BH, Nk, &krows))
        return ATTN_BAD_SHAPE;
    // 2. Head dimension.
    if (d != 64 && d != 128)
        return ATTN_UNSUPPORTED_D;
    if (!mul_ok(qrows, d, &qelems) || !mul_ok(qelems, 2, &qbytes) || !mul_ok(krows, d, &kelems) ||
        !mul_ok(kelems, 2, &kbytes) || !mul_ok(qrows, 4, &lse_bytes))
        return ATTN_BAD_SHAPE;
    if (Nq * d >= (int64_t(1) << 31) || Nk * d >= (int64_t(1) << 31))  // in-head offsets are 32-bit
        return ATTN_BAD_SHAPE;
    if (qrows > 0 && (Nk == 0 || (causal && Nq > Nk)))  // a query with no key to attend to
        return ATTN_BAD_SHAPE;
    if (qrows > 0 && attn_workgroups(BH, Nq, Nk, num_splits) > INT32_MAX)
        return ATTN_BAD_SHAPE;
    const int64_t splits = qrows > 0 ? attn_splits_used(Nk, num_splits) : 1;
    int64_t ws_need = 0;
    if (splits > 1) {
        int64_t t;
        if (!mul_ok(splits, qrows, &t) || !mul_ok(t, d + 1, &t) || !mul_ok(t, 4, &ws_need))
            return ATTN_BAD_SHAPE;
        if (qrows * (d / 8) > INT32_MAX - 255)  // one merge thread per 8 columns of a row
            return ATTN_BAD_SHAPE;
    }
    // 3. Scale.
    if (!std::isfinite(scale))
        return ATTN_BAD_SCALE;
    // 4. Empty problem: nothing to read or write.
    if (qrows == 0)
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
    if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) || overlaps(o, qbytes, v, kbytes))
        return ATTN_ALIAS;
    if (lse && (overlaps(lse, lse_bytes, q, qbytes) || overlaps(lse, lse_bytes, k, kbytes) ||
                overlaps(lse, lse_bytes, v, kbytes) || overlaps(lse, lse_bytes, o, qbytes)))
        return ATTN_ALIAS;
    // 8. Workspace (split ranges only): the caller's, or the library's scratch.
    if (splits > 1 && use_scratch) {
        if (ws_need > kScratchBytes)
            return ATTN_SCRATCH_TOO_SMALL;
        const hipError_t err = scratch_address(&workspace);
        if (err != hipSuccess) {
            g_last_hip_error = static_cast<int>(err);
            return ATTN_HIP;
        }
    } else if (splits > 1) {
        if (!workspace || mis16(workspace) || workspace_bytes < ws_need ||
            overlaps(workspace, ws_need, q, qbytes) || overlaps(workspace, ws_need, k, kbytes) ||
            overlaps(workspace, ws_need, v, kbytes) || overlaps(workspace, ws_need, o, qbytes) ||
            (lse && overlaps(workspace, ws_need, lse, lse_bytes)))
            return ATTN_BAD_WORKSPACE;
    }

    AttnLaunch a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.BH = BH;
    a.Nq = Nq;
    a.Nk = Nk;
    a.d = d;
    a.causal = causal != 0;
    a.scale = scale;
    a.num_splits = num_splits;
    a.workspace = splits > 1 ? workspace : nullptr;
    a.stream = static_cast<hipStream_t>(stream);
    const hipError_t err = attn_launch(a);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return ATTN_HIP;
    }
    return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                        void *stream)
{
    return fwd_common(q, k, v, o, lse, B, H, N, N, d, causal, scale, 1, nullptr, 0, stream);
}

extern "C" int attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                                int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                                float scale, int64_t num_splits, void *workspace, int64_t workspace_bytes,
                                void *stream)
{
    return fwd_common(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, workspace,
                      workspace_bytes, stream);
}

extern "C" int attn_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                                        float scale, int64_t num_splits, void *stream)
{
    return fwd_common(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, num_splits, nullptr, 0, stream, true);
}

extern "C" int64_t attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int64_t attn_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t d,
                                                    int64_t num_splits)
{
    int64_t BH, rows, t, bytes;
    if (B < 0 || H < 0 || Nq < 0 || num_splits < 1 || (d != 64 && d != 128) || !mul_ok(B, H, &BH) ||
        !mul_ok(BH, Nq, &rows))
        return -1;
    if (num_splits == 1)
        return 0;
    if (!mul_ok(num_splits, rows, &t) || !mul_ok(t, d + 1, &t) || !mul_ok(t, 4, &bytes))
        return -1;
    return bytes;
}

extern "C" int64_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d)
{
    int64_t BH, rows, bytes;
    if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128) || !mul_ok(B, H, &BH) || !mul_ok(BH, N, &rows) ||
        !mul_ok(rows, 8, &bytes))
        return -1;
    return bytes;
}

extern "C" int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H, int64_t N,
                        int64_t d, int causal, float scale, void *workspace, int64_t workspace_bytes,
                        void *stream)
{
    // 1. Shapes.
    int64_t BH, rows, elems, bytes, vec_bytes, ws_need;
    if (B < 0 || H < 0 || N < 0 || !mul_ok(B, H, &BH) || !mul_ok(BH, N, &rows))
        return ATTN_BAD_SHAPE;
    // 2. Head dimension.
    if (d != 64 && d != 128)
        return ATTN_UNSUPPORTED_D;
    if (!mul_ok(rows, d, &elems) || !mul_ok(elems, 2, &bytes) || !mul_ok(rows, 4, &vec_bytes) ||
        !mul_ok(rows, 8, &ws_need))
        return ATTN_BAD_SHAPE;
    if (N * d >= (int64_t(1) << 31))  // in-head offsets are 32-bit
        return ATTN_BAD_SHAPE;
    if (rows > 0 && attn_bwd_workgroups(BH, N) > INT32_MAX)
        return ATTN_BAD_SHAPE;
    // 3. Scale.
    if (!std::isfinite(scale))
        return ATTN_BAD_SCALE;
    // 4. Empty problem.
    if (rows == 0)
        return ATTN_OK;
    // 5. Pointers.
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
        return ATTN_NULL_PTR;
    // 6. Alignment.
    const auto mis16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
    if (mis16(q) || mis16(k) || mis16(v) || mis16(o) || mis16(dout) || mis16(dq) || mis16(dk) || mis16(dv) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
        return ATTN_MISALIGNED;
    // 7. Outputs must not overlap any input or each other (inputs may alias
    //    one another).
    const void *ins[6] = {q, k, v, o, dout, lse};
    const int64_t in_bytes[6] = {bytes, bytes, bytes, bytes, bytes, vec_bytes};
    void *outs[3] = {dq, dk, dv};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], bytes, ins[j], in_bytes[j]))
                return ATTN_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], bytes, outs[j], bytes))
                return ATTN_ALIAS;
    }
    // 8. Workspace.
    if (!workspace || mis16(workspace) || workspace_bytes < ws_need)
        return ATTN_BAD_WORKSPACE;
    for (int j = 0; j < 6; ++j)
        if (overlaps(workspace, ws_need, ins[j], in_bytes[j]))
            return ATTN_BAD_WORKSPACE;
    for (int i = 0; i < 3; ++i)
        if (overlaps(workspace, ws_need, outs[i], bytes))
            return ATTN_BAD_WORKSPACE;

    AttnBwdLaunch a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.workspace = workspace;
    a.BH = BH;
    a.N = N;
    a.d = d;
    a.causal = causal != 0;
    a.scale = scale;
    a.stream = static_cast<hipStream_t>(stream);
    const hipError_t err = attn_bwd_launch(a);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return ATTN_HIP;
    }
    return ATTN_OK;
}

extern "C" int64_t attn_fp8_padded_rows(int64_t N) { return N < 0 ? -1 : attn_fp8_rows(N); }

// attn_fp8_quantize and attn_fp8_quantize_q: `scale` is null for the first
// (no multiplier), else the softmax scale of Q's call.
static int fp8_quantize(const void *x, int64_t B, int64_t H, int64_t N, int64_t d, int transpose,
                        const uint32_t *sign_bits, const float *scale, void *out, void *exps, void *stream)
{
    int64_t BH, rows, np_rows, bytes, xbytes, nexp;
    if (B < 0 || H < 0 || N < 0 || !mul_ok(B, H, &BH) || !mul_ok(BH, N, &rows))
        return ATTN_BAD_SHAPE;
    if (d != 128)
        return ATTN_UNSUPPORTED_D;
    const int64_t Np = attn_fp8_rows(N);
    if (!mul_ok(BH, Np, &np_rows) || !mul_ok(np_rows, d, &bytes) || !mul_ok(rows, 2 * d, &xbytes) ||
        N * d >= (int64_t(1) << 31) || Np * d >= (int64_t(1) << 31) || np_rows / 64 > INT32_MAX)
        return ATTN_BAD_SHAPE;
    nexp = np_rows / 64;
    if (transpose && sign_bits)  // V is not rotated
        return ATTN_BAD_ARGUMENT;
    if (scale && !std::isfinite(*scale))
        return ATTN_BAD_SCALE;
    if (rows == 0)
        return ATTN_OK;
    if (!x || !out || !exps)
        return ATTN_NULL_PTR;
    if ((reinterpret_cast<uintptr_t>(x) & 15u) || (reinterpret_cast<uintptr_t>(out) & 15u))
        return ATTN_MISALIGNED;
    if (overlaps(out, bytes, x, xbytes) || overlaps(exps, nexp, x, xbytes) || overlaps(exps, nexp, out, bytes))
        return ATTN_ALIAS;
    AttnFp8Quantize q;
    q.x = x;
    q.out = out;
    q.exps = exps;
    q.sign_bits = sign_bits;
    q.transpose = transpose != 0;
    // Q's logits in log2 units: scale * log2(e), and 1/d when Q and K are
    // rotated (their product then carries the Hadamard factor d); one fp32
    // product, then an exact power of two.
    q.mul = 1.f;
    if (scale) {
        q.mul = *scale * attn_gfx950::kLog2e;
        if (sign_bits)
            q.mul *= 1.f / static_cast<float>(d);
    }
    q.BH = BH;
    q.N = N;
    q.stream = static_cast<hipStream_t>(stream);
    const hipError_t err = attn_fp8_quantize_launch(q);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return ATTN_HIP;
    }
    return ATTN_OK;
}

extern "C" int attn_fp8_quantize(const void *x, int64_t B, int64_t H, int64_t N, int64_t d, int transpose,
                                 const uint32_t *sign_bits, void *out, void *exps, void *stream)
{
    return fp8_quantize(x, B, H, N, d, transpose, sign_bits, nullptr, out, exps, stream);
}

extern "C" int attn_fp8_quantize_q(const void *x, int64_t B, int64_t H, int64_t N, int64_t d,
                                   const uint32_t *sign_bits, float scale, void *out, void *exps, void *stream)
{
    return fp8_quantize(x, B, H, N, d, 0, sign_bits, &scale, out, exps, stream);
}

extern "C" int attn_fwd_fp8(const void *q8, const void *k8, const void *vt8, const void *q_exps, const void *k_exps,
                            const void *v_exps, void *o, float *lse, int64_t B, int64_t H, int64_t N, int64_t d,
                            int causal, void *stream)
{
    int64_t BH, rows, np_rows, bytes, obytes, lse_bytes, nexp;
    if (B < 0 || H < 0 || N < 0 || !mul_ok(B, H, &BH) || !mul_ok(BH, N, &rows))
        return ATTN_BAD_SHAPE;
    if (d != 128)
        return ATTN_UNSUPPORTED_D;
    const int64_t Np = attn_fp8_rows(N);
    if (!mul_ok(BH, Np, &np_rows) || !mul_ok(np_rows, d, &bytes) || !mul_ok(rows, 2 * d, &obytes) ||
        !mul_ok(rows, 4, &lse_bytes) || N * d >= (int64_t(1) << 31) || Np * d >= (int64_t(1) << 31) ||
        attn_workgroups(BH, N, N, 1) > INT32_MAX)
        return ATTN_BAD_SHAPE;
    nexp = np_rows / 64;
    if (rows == 0)
        return ATTN_OK;
    if (!q8 || !k8 || !vt8 || !q_exps || !k_exps || !v_exps || !o)
        return ATTN_NULL_PTR;
    const auto mis16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
    if (mis16(q8) || mis16(k8) || mis16(vt8) || mis16(o) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return ATTN_MISALIGNED;
    const void *ins[6] = {q8, k8, vt8, q_exps, k_exps, v_exps};
    const int64_t in_bytes[6] = {bytes, bytes, bytes, nexp, nexp, nexp};
    for (int j = 0; j < 6; ++j)
        if (overlaps(o, obytes, ins[j], in_bytes[j]) || (lse && overlaps(lse, lse_bytes, ins[j], in_bytes[j])))
            return ATTN_ALIAS;
    if (lse && overlaps(lse, lse_bytes, o, obytes))
        return ATTN_ALIAS;
    AttnFp8Launch a;
    a.q8 = q8;
    a.k8 = k8;
    a.vt8 = vt8;
    a.qe = q_exps;
    a.ke = k_exps;
    a.ve = v_exps;
    a.o = o;
    a.lse = lse;
    a.BH = BH;
    a.N = N;
    a.causal = causal != 0;
    a.stream = static_cast<hipStream_t>(stream);
    const hipError_t err = attn_fp8_launch(a);
    if (err != hipSuccess) {
        g_last_hip_error = static_cast<int>(err);
        return ATTN_HIP;
    }
    return ATTN_OK;
}
