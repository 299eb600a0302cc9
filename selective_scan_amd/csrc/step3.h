// Host-side declarations of the Mamba-3 one-token decode step (step3.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "launch.h"

namespace ssm {

struct Step3Args {
    int B, D, N;
    bool bf16;
    float* state;        // [B, D, N, 2] complex (real, imaginary), updated in place
    const void* x;       // [B, D]
    const void* delta;   // [B, D]
    const void* lam;     // [B, D]
    const float* Are;    // [D, N]
    const float* theta;  // [D, N]
    const void* Bm;      // [B, N]
    const void* Cm;      // [B, N]
    const float* Dskip;  // [D] or NULL
    const void* z;       // [B, D] or NULL
    const void* x_prev;  // [B, D] or NULL (with B_prev: the previous token)
    const void* B_prev;  // [B, N] or NULL
    void* y;             // [B, D]
};

bool step3_supported_n(int N);
hipError_t launch_step3(const Step3Args& a, hipStream_t stream);

}  // namespace ssm
