// Host-side declarations of the Mamba-3 scan (scan3.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "launch.h"

namespace ssm {

struct Scan3Args {
    int B, L, D, N;
    bool bf16;
    const void* x;
    const void* delta;
    const void* lam;
    const float* Are;
    const float* theta;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const void* z;
    const float* h0;  // [B, D, N, 2] complex (real, imaginary) or NULL
    const void* x_prev;
    const void* B_prev;
    void* y;
    float* h_final;   // [B, D, N, 2] or NULL
    void* ws;
};

bool scan3_supported_n(int N);
int scan3_segment_len(int B, int L, int D);
size_t scan3_workspace_bytes(int B, int L, int D, int N);
hipError_t launch_scan3_fwd(const Scan3Args& a, hipStream_t stream);

}  // namespace ssm
