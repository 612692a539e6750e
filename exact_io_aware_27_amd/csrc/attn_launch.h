// attn_launch.h -- internal interface between the validating C ABI
// (attn_api.hip) and the gfx950 kernels (attn_fwd_kernel.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Arguments of one validated attn_fwd call.  Sizes are already checked:
// d is 64 or 128, N * d < 2^31, and the workgroup count fits in an int.
struct AttnLaunch {
    const void *q, *k, *v;
    void *o;
    float *lse;  // may be null
    int64_t BH, N, d;
    bool causal;
    float scale;
    hipStream_t stream;
};

// An upper bound on the workgroups one call launches for B*H heads of length N.
int64_t attn_workgroups(int64_t BH, int64_t N);

// Enqueue the kernel; returns hipGetLastError() after the launch.
hipError_t attn_launch(const AttnLaunch &a);
