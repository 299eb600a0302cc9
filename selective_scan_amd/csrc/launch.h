// Host-side launchers of the gfx950 kernels (internal to the library; the C ABI
// in api.cpp validates arguments and then calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <stddef.h>

namespace ssm {

// The next two caller-provided timing events if the calling thread enabled
// ssm_profile_events() and two remain; otherwise both null.
void profile_events(hipEvent_t* start, hipEvent_t* stop);

// Launches `kernel` on `stream`. When timing is on, the runtime stamps the two
// events at the kernel's own start and end (not at the surrounding queue
// positions), so the pair times the kernel alone.
template <typename... Params, typename... Args>
inline void launch(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t lds, hipStream_t stream,
                   Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    profile_events(&e0, &e1);
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, e0, e1, 0u, static_cast<Params>(args)...);
}

// ------------------------------------------------------------ Mamba-1 scan
struct ScanArgs {
    int B, L, D, N;
    bool bf16;
    const void* x;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const void* z;
    const float* h0;
    void* y;
    float* h_final;
    void* ws;
    // discretisation variant (ssm_scan_fwd_ex): 0 exponential-Euler, 1 zero-order
    // hold; Delta = [softplus](delta + delta_bias) when either is set
    const float* delta_bias;
    int delta_softplus;
    int disc;
};

// How the sequence is cut for the L-parallel scan: S segments of Ls steps
// (the last one may be shorter). Depends only on the shape.
struct ScanPlan {
    int S;
    int Ls;
};

bool scan_supported_n(int N);
ScanPlan scan_plan(int B, int L, int D, int N);
size_t scan_workspace_bytes(int B, int L, int D, int N);
hipError_t launch_scan_fwd(const ScanArgs& a, hipStream_t stream);
// zero-order hold and/or Delta preprocessing; N in {4, 8, 16, 32}
bool scan_var_supported_n(int N);
hipError_t launch_scan_fwd_var(const ScanArgs& a, hipStream_t stream);

// ------------------------------------------------------------ Mamba-1 scan, backward
struct BwdArgs {
    int B, L, D, N;
    bool bf16;
    const void* x;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const void* z;
    const float* h0;
    const void* dy;
    const float* dh_final;
    void* dx;
    void* ddelta;
    float* dA;
    void* dBm;
    void* dCm;
    float* dDskip;
    void* dz;
    float* dh0;
    void* ws;
};

bool scan_bwd_supported_n(int N);
int scan_bwd_segment_len(int B, int L, int D, int N);
size_t scan_bwd_workspace_bytes(int B, int L, int D, int N);
hipError_t launch_scan_bwd(const BwdArgs& a, hipStream_t stream);

// ------------------------------------------------------------ decode step
struct StepArgs {
    int B, D, N;
    bool bf16;
    float* state;
    const void* x;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const void* z;
    void* y;
    // discretisation variant (ssm_step_ex), as in ScanArgs
    const float* delta_bias;
    int delta_softplus;
    int disc;
};

bool step_supported_n(int N);
hipError_t launch_step(const StepArgs& a, hipStream_t stream);
hipError_t launch_step_var(const StepArgs& a, hipStream_t stream);

// ------------------------------------------------------------ SSD decode step
struct SsdStepArgs {
    int B, H, P, N;
    bool bf16;
    float* state;
    const void* x;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const void* z;
    void* y;
};

bool ssd_step_supported(int P, int N);
hipError_t launch_ssd_step(const SsdStepArgs& a, hipStream_t stream);

// ------------------------------------------------------------ SSD
struct SsdArgs {
    int B, L, H, P, N, Q;
    bool bf16;
    const void* x;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const void* z;
    const float* h0;
    void* y;
    float* h_final;
    void* ws;
};

// Returns an empty string when the shape is supported, else the reason.
const char* ssd_unsupported_reason(int L, int H, int P, int N, int Q, bool bf16);
size_t ssd_workspace_bytes(int B, int L, int H, int P, int N, int Q);
hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t stream);

}  // namespace ssm
