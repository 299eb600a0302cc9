// C ABI of the selective-scan library: argument validation (before any HIP call),
// status codes and dispatch to the gfx950 launchers. Declared in include/ssm_scan.h.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <string>

#include "extras.h"
#include "launch.h"
#include "scan3.h"
#include "step3.h"

namespace {

thread_local std::string g_last_error;

struct ProfileEvents {
    void* const* ev = nullptr;
    int n = 0;
    int used = 0;
};
thread_local ProfileEvents g_prof;

int fail(int status, const char* fn, const char* what) {
    g_last_error = std::string(fn) + ": " + what;
    return status;
}

int ok() {
    g_last_error.clear();
    return SSM_OK;
}

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// n1*n2*... fits in int64 without overflow
bool product_ok(std::initializer_list<long long> dims, long long limit = std::numeric_limits<long long>::max()) {
    long long p = 1;
    for (long long d : dims) {
        if (d < 0) return false;
        if (d != 0 && p > limit / d) return false;
        p *= d;
    }
    return true;
}

int hip_status(hipError_t e, const char* fn) {
    if (e == hipSuccess) return ok();
    char buf[256];
    std::snprintf(buf, sizeof buf, "HIP error %d (%s)", (int)e, hipGetErrorString(e));
    return fail(SSM_ERR_HIP, fn, buf);
}

}  // namespace

namespace ssm {
void profile_events(hipEvent_t* start, hipEvent_t* stop) {
    *start = *stop = nullptr;
    if (g_prof.ev == nullptr || g_prof.used + 2 > g_prof.n) return;
    *start = static_cast<hipEvent_t>(g_prof.ev[g_prof.used]);
    *stop = static_cast<hipEvent_t>(g_prof.ev[g_prof.used + 1]);
    g_prof.used += 2;
}
}  // namespace ssm

extern "C" {

int ssm_profile_events(void* const* events, int n) {
    const int used = g_prof.used;
    g_prof.ev = (events != nullptr && n > 0) ? events : nullptr;
    g_prof.n = g_prof.ev ? n : 0;
    g_prof.used = 0;
    return used;
}

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(int s) {
    switch (s) {
        case SSM_OK: return "SSM_OK";
        case SSM_ERR_INVALID_ARG: return "SSM_ERR_INVALID_ARG";
        case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED";
        case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE";
        case SSM_ERR_HIP: return "SSM_ERR_HIP";
        default: return "SSM_ERR_UNKNOWN";
    }
}

const char* ssm_last_error(void) { return g_last_error.c_str(); }

// ------------------------------------------------------------------ scan
size_t ssm_scan_workspace_size(int B, int L, int D, int N) {
    if (B < 1 || L < 0 || D < 1 || !ssm::scan_supported_n(N)) return 0;
    if (!product_ok({B, L, D, N})) return 0;
    return ssm::scan_workspace_bytes(B, L, D, N);
}

}  // extern "C"

namespace {

// ssm_scan_fwd and ssm_scan_fwd_ex: validation, then the plain or the variant path.
int scan_fwd_impl(const char* fn, int B, int L, int D, int N, int io, int disc, const float* delta_bias,
                  int delta_softplus, const void* x, const void* delta, const float* A, const void* Bm,
                  const void* Cm, const float* Dskip, const void* z, const float* h0, void* y, float* h_final,
                  void* workspace, size_t workspace_bytes, void* stream, bool launch = true) {
    if (B < 1 || D < 1 || L < 0 || N < 1) return fail(SSM_ERR_INVALID_ARG, fn, "B, D, N must be >= 1 and L >= 0");
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, fn, "io must be SSM_F32 or SSM_BF16");
    if (disc != SSM_DISC_EULER && disc != SSM_DISC_ZOH)
        return fail(SSM_ERR_INVALID_ARG, fn, "disc must be SSM_DISC_EULER or SSM_DISC_ZOH");
    const bool variant = disc != SSM_DISC_EULER || delta_bias != nullptr || delta_softplus != 0;
    if (!ssm::scan_supported_n(N)) return fail(SSM_ERR_UNSUPPORTED, fn, "N must be one of 4, 8, 16, 32, 64, 128, 256");
    if (variant && !ssm::scan_var_supported_n(N))
        return fail(SSM_ERR_UNSUPPORTED, fn, "zero-order hold and Delta preprocessing: unsupported N");
    if (B > 65535) return fail(SSM_ERR_UNSUPPORTED, fn, "B must be <= 65535");
    if (!product_ok({B, L, D, N}) || !product_ok({B, L, D}, 1LL << 40))
        return fail(SSM_ERR_INVALID_ARG, fn, "tensor sizes overflow");
    if (!A) return fail(SSM_ERR_INVALID_ARG, fn, "A is NULL");
    if (L > 0 && (!x || !delta || !Bm || !Cm || !y))
        return fail(SSM_ERR_INVALID_ARG, fn, "x, delta, Bm, Cm and y are required");
    const void* ptrs[] = {x, delta, A, Bm, Cm, Dskip, z, h0, y, h_final, workspace, delta_bias};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SSM_ERR_INVALID_ARG, fn, "every pointer must be 16-byte aligned");
    const int es = io == SSM_BF16 ? 2 : 4;
    const ssm::ScanPlan plan = ssm::scan_plan(B, L, D, N);
    if ((long long)plan.Ls * D * es >= (1LL << 31))
        return fail(SSM_ERR_UNSUPPORTED, fn, "one segment of [L, D] exceeds 2 GiB");
    const size_t need = ssm::scan_workspace_bytes(B, L, D, N);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(SSM_ERR_WORKSPACE, fn, "workspace missing or smaller than ssm_scan_workspace_size()");
    if (!launch) return ok();
    ssm::ScanArgs a{B, L, D, N, io == SSM_BF16, x, delta, A, Bm, Cm, Dskip, z, h0, y, h_final, workspace,
                    delta_bias, delta_softplus, disc};
    const hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(variant ? ssm::launch_scan_fwd_var(a, st) : ssm::launch_scan_fwd(a, st), fn);
}

// ssm_step and ssm_step_ex
int step_impl(const char* fn, int B, int D, int N, int io, int disc, const float* delta_bias, int delta_softplus,
              float* state, const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
              const float* Dskip, const void* z, void* y, void* stream) {
    if (B < 1 || D < 1 || N < 1) return fail(SSM_ERR_INVALID_ARG, fn, "B, D, N must be >= 1");
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, fn, "io must be SSM_F32 or SSM_BF16");
    if (disc != SSM_DISC_EULER && disc != SSM_DISC_ZOH)
        return fail(SSM_ERR_INVALID_ARG, fn, "disc must be SSM_DISC_EULER or SSM_DISC_ZOH");
    if (!ssm::step_supported_n(N)) return fail(SSM_ERR_UNSUPPORTED, fn, "N must be one of 4, 8, 16, 32, 64, 128, 256");
    if (B > 65535) return fail(SSM_ERR_UNSUPPORTED, fn, "B must be <= 65535");
    if (!product_ok({B, D, N}, 1LL << 40)) return fail(SSM_ERR_INVALID_ARG, fn, "tensor sizes overflow");
    if ((long long)D * N > (1LL << 32)) return fail(SSM_ERR_UNSUPPORTED, fn, "D * N must be <= 2^32");
    if (!state || !x || !delta || !A || !Bm || !Cm || !y)
        return fail(SSM_ERR_INVALID_ARG, fn, "state, x, delta, A, Bm, Cm and y are required");
    const void* ptrs[] = {state, x, delta, A, Bm, Cm, Dskip, z, y, delta_bias};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SSM_ERR_INVALID_ARG, fn, "every pointer must be 16-byte aligned");
    ssm::StepArgs a{B, D, N, io == SSM_BF16, state, x, delta, A, Bm, Cm, Dskip, z, y,
                    delta_bias, delta_softplus, disc};
    const bool variant = disc != SSM_DISC_EULER || delta_bias != nullptr || delta_softplus != 0;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(variant ? ssm::launch_step_var(a, st) : ssm::launch_step(a, st), fn);
}

// The SSD chunk length the kernels run: 256 by default; chunks above 256 steps (one
// chunk's rows must fit a workgroup's LDS) run as 256-step chunks. The chunked form
// computes the same recurrence whatever its chunk length; only the rounding follows
// the chunking.
int ssd_chunk(int chunk) { return chunk == 0 ? 256 : std::min(chunk, 256); }

}  // namespace

extern "C" {

int ssm_scan_fwd(int B, int L, int D, int N, ssm_dtype_t io,
                 const void* x, const void* delta, const float* A,
                 const void* Bm, const void* Cm, const float* Dskip,
                 const void* z, const float* h0,
                 void* y, float* h_final,
                 void* workspace, size_t workspace_bytes, void* stream) {
    return scan_fwd_impl("ssm_scan_fwd", B, L, D, N, io, SSM_DISC_EULER, nullptr, 0, x, delta, A, Bm, Cm, Dskip,
                         z, h0, y, h_final, workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_ex(int B, int L, int D, int N, ssm_dtype_t io, ssm_disc_t disc,
                    const float* delta_bias, int delta_softplus,
                    const void* x, const void* delta, const float* A,
                    const void* Bm, const void* Cm, const float* Dskip,
                    const void* z, const float* h0,
                    void* y, float* h_final,
                    void* workspace, size_t workspace_bytes, void* stream) {
    return scan_fwd_impl("ssm_scan_fwd_ex", B, L, D, N, io, disc, delta_bias, delta_softplus, x, delta, A, Bm,
                         Cm, Dskip, z, h0, y, h_final, workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_noalloc(int B, int L, int D, int N, ssm_dtype_t io,
                         const void* x, const void* delta, const float* A,
                         const void* Bm, const void* Cm, const float* Dskip,
                         const void* z, const float* h0,
                         void* y, float* h_final, void* stream) {
    const char* fn = "ssm_scan_fwd_noalloc";
    // the checks of ssm_scan_fwd, then the size limit of the fixed scratch, all
    // before any HIP call
    const size_t need = (B >= 1 && D >= 1 && L >= 0 && ssm::scan_supported_n(N) && product_ok({B, L, D, N}))
                            ? ssm::scan_workspace_bytes(B, L, D, N)
                            : 0;
    // a stand-in workspace address of exactly the needed size (never dereferenced:
    // scan_fwd_impl only validates here)
    void* stand_in = need > 0 ? reinterpret_cast<void*>(uintptr_t{256}) : nullptr;
    const int st = scan_fwd_impl(fn, B, L, D, N, io, SSM_DISC_EULER, nullptr, 0, x, delta, A, Bm, Cm, Dskip, z, h0,
                                 y, h_final, stand_in, need, nullptr, /*launch=*/false);
    if (st != SSM_OK) return st;
    if (need > ssm::kNoallocScratchBytes) {
        char buf[160];
        std::snprintf(buf, sizeof buf, "the shape needs %zu bytes of scratch; the fixed scratch holds %zu", need,
                      ssm::kNoallocScratchBytes);
        return fail(SSM_ERR_UNSUPPORTED, fn, buf);
    }
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    int dev = -1;
    hipError_t e = hs ? hipStreamGetDevice(hs, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    void* ws = nullptr;
    if ((e = ssm::noalloc_scratch(dev, &ws)) != hipSuccess) return hip_status(e, fn);
    ssm::ScanArgs a{B, L, D, N, io == SSM_BF16, x, delta, A, Bm, Cm, Dskip, z, h0, y, h_final, ws,
                    nullptr, 0, SSM_DISC_EULER};
    return hip_status(ssm::launch_scan_fwd(a, hs), fn);
}

// ------------------------------------------------------------------ Mamba-3 scan
size_t ssm_scan3_workspace_size(int B, int L, int D, int N) {
    if (B < 1 || L < 0 || D < 1 || !ssm::scan3_supported_n(N)) return 0;
    if (!product_ok({B, L, D, N})) return 0;
    return ssm::scan3_workspace_bytes(B, L, D, N);
}

int ssm_scan3_fwd(int B, int L, int D, int N, ssm_dtype_t io,
                  const void* x, const void* delta, const void* lam,
                  const float* Are, const float* theta,
                  const void* Bm, const void* Cm, const float* Dskip, const void* z,
                  const float* h0, const void* x_prev, const void* B_prev,
                  void* y, float* h_final,
                  void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ssm_scan3_fwd";
    if (B < 1 || D < 1 || L < 0 || N < 1) return fail(SSM_ERR_INVALID_ARG, fn, "B, D, N must be >= 1 and L >= 0");
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, fn, "io must be SSM_F32 or SSM_BF16");
    if (!ssm::scan3_supported_n(N)) return fail(SSM_ERR_UNSUPPORTED, fn, "N must be one of 4, 8, 16");
    if (B > 65535) return fail(SSM_ERR_UNSUPPORTED, fn, "B must be <= 65535");
    if (!product_ok({B, L, D, N}, 1LL << 40) || !product_ok({B, L, D}, 1LL << 40))
        return fail(SSM_ERR_INVALID_ARG, fn, "tensor sizes overflow");
    if (!Are || !theta) return fail(SSM_ERR_INVALID_ARG, fn, "Are and theta are required");
    if (L > 0 && (!x || !delta || !lam || !Bm || !Cm || !y))
        return fail(SSM_ERR_INVALID_ARG, fn, "x, delta, lam, Bm, Cm and y are required");
    if ((x_prev == nullptr) != (B_prev == nullptr))
        return fail(SSM_ERR_INVALID_ARG, fn, "x_prev and B_prev must be given together");
    const void* ptrs[] = {x, delta, lam, Are, theta, Bm, Cm, Dskip, z, h0, x_prev, B_prev, y, h_final, workspace};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SSM_ERR_INVALID_ARG, fn, "every pointer must be 16-byte aligned");
    const size_t need = ssm::scan3_workspace_bytes(B, L, D, N);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(SSM_ERR_WORKSPACE, fn, "workspace missing or smaller than ssm_scan3_workspace_size()");
    ssm::Scan3Args a{B, L, D, N, io == SSM_BF16, x, delta, lam, Are, theta, Bm, Cm, Dskip, z, h0, x_prev, B_prev,
                     y, h_final, workspace};
    return hip_status(ssm::launch_scan3_fwd(a, static_cast<hipStream_t>(stream)), fn);
}

int ssm_step3(int B, int D, int N, ssm_dtype_t io,
              float* state, const void* x, const void* delta, const void* lam,
              const float* Are, const float* theta, const void* Bm, const void* Cm,
              const float* Dskip, const void* z, const void* x_prev, const void* B_prev,
              void* y, void* stream) {
    const char* fn = "ssm_step3";
    if (B < 1 || D < 1 || N < 1) return fail(SSM_ERR_INVALID_ARG, fn, "B, D, N must be >= 1");
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, fn, "io must be SSM_F32 or SSM_BF16");
    if (!ssm::step3_supported_n(N)) return fail(SSM_ERR_UNSUPPORTED, fn, "N must be one of 4, 8, 16, 32, 64, 128");
    if (B > 65535) return fail(SSM_ERR_UNSUPPORTED, fn, "B must be <= 65535");
    if ((long long)D * N > 0x7fffffffLL) return fail(SSM_ERR_UNSUPPORTED, fn, "D * N must be < 2^31");
    if (!product_ok({B, D, N}, 1LL << 40)) return fail(SSM_ERR_INVALID_ARG, fn, "tensor sizes overflow");
    if (!state || !x || !delta || !lam || !Are || !theta || !Bm || !Cm || !y)
        return fail(SSM_ERR_INVALID_ARG, fn, "state, x, delta, lam, Are, theta, Bm, Cm and y are required");
    if ((x_prev == nullptr) != (B_prev == nullptr))
        return fail(SSM_ERR_INVALID_ARG, fn, "x_prev and B_prev must be given together");
    const void* ptrs[] = {state, x, delta, lam, Are, theta, Bm, Cm, Dskip, z, x_prev, B_prev, y};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SSM_ERR_INVALID_ARG, fn, "every pointer must be 16-byte aligned");
    ssm::Step3Args a{B, D, N, io == SSM_BF16, state, x, delta, lam, Are, theta, Bm, Cm, Dskip, z, x_prev, B_prev, y};
    return hip_status(ssm::launch_step3(a, static_cast<hipStream_t>(stream)), fn);
}

// ------------------------------------------------------------------ scan backward
size_t ssm_scan_bwd_workspace_size(int B, int L, int D, int N) {
    if (B < 1 || L < 0 || D < 1 || !ssm::scan_bwd_supported_n(N)) return 0;
    if (!product_ok({B, L, D, N})) return 0;
    return ssm::scan_bwd_workspace_bytes(B, L, D, N);
}

int ssm_scan_bwd(int B, int L, int D, int N, ssm_dtype_t io,
                 const void* x, const void* delta, const float* A,
                 const void* Bm, const void* Cm, const float* Dskip,
                 const void* z, const float* h0,
                 const void* dy, const float* dh_final,
                 void* dx, void* ddelta, float* dA, void* dBm, void* dCm,
                 float* dDskip, void* dz, float* dh0,
                 void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ssm_scan_bwd";
    if (B < 1 || D < 1 || L < 0 || N < 1) return fail(SSM_ERR_INVALID_ARG, fn, "B, D, N must be >= 1 and L >= 0");
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, fn, "io must be SSM_F32 or SSM_BF16");
    if (!ssm::scan_bwd_supported_n(N)) return fail(SSM_ERR_UNSUPPORTED, fn, "N must be one of 4, 8, 16, 32, 64, 128, 256");
    if (B > 65535) return fail(SSM_ERR_UNSUPPORTED, fn, "B must be <= 65535");
    if (!product_ok({B, L, D, N}, 1LL << 40) || !product_ok({B, L, D}, 1LL << 40))
        return fail(SSM_ERR_INVALID_ARG, fn, "tensor sizes overflow");
    if (!A || !dA) return fail(SSM_ERR_INVALID_ARG, fn, "A and dA are required");
    if (L > 0 && (!x || !delta || !Bm || !Cm || !dy || !dx || !ddelta || !dBm || !dCm))
        return fail(SSM_ERR_INVALID_ARG, fn, "x, delta, Bm, Cm, dy, dx, ddelta, dBm and dCm are required");
    if ((Dskip == nullptr) != (dDskip == nullptr))
        return fail(SSM_ERR_INVALID_ARG, fn, "dDskip must be given exactly when Dskip is");
    if ((z == nullptr) != (dz == nullptr))
        return fail(SSM_ERR_INVALID_ARG, fn, "dz must be given exactly when z is");
    const void* ptrs[] = {x, delta, A, Bm, Cm, Dskip, z, h0, dy, dh_final, dx, ddelta,
                          dA, dBm, dCm, dDskip, dz, dh0, workspace};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SSM_ERR_INVALID_ARG, fn, "every pointer must be 16-byte aligned");
    const int es = io == SSM_BF16 ? 2 : 4;
    const long long Ls = ssm::scan_bwd_segment_len(B, L, D, N);
    if (Ls * D * es >= (1LL << 31) || Ls * N * 4 >= (1LL << 31))
        return fail(SSM_ERR_UNSUPPORTED, fn, "one segment of [L, D] exceeds 2 GiB");
    const size_t need = ssm::scan_bwd_workspace_bytes(B, L, D, N);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(SSM_ERR_WORKSPACE, fn, "workspace missing or smaller than ssm_scan_bwd_workspace_size()");
    ssm::BwdArgs a{B, L, D, N, io == SSM_BF16, x, delta, A, Bm, Cm, Dskip, z, h0, dy, dh_final,
                   dx, ddelta, dA, dBm, dCm, dDskip, dz, dh0, workspace};
    return hip_status(ssm::launch_scan_bwd(a, static_cast<hipStream_t>(stream)), fn);
}

// ------------------------------------------------------------------ SSD
size_t ssm_ssd_workspace_size(int B, int L, int H, int P, int N, int chunk) {
    const int Q = ssd_chunk(chunk);
    if (B < 1 || L < 0 || H < 1 || P < 1 || N < 1 || Q < 1) return 0;
    if (!product_ok({B, L, H, P}) || !product_ok({B, H, N, P})) return 0;
    return ssm::ssd_workspace_bytes(B, L, H, P, N, Q);
}

int ssm_ssd_fwd(int B, int L, int H, int P, int N, int chunk, ssm_dtype_t io,
                const void* x, const void* delta, const float* A,
                const void* Bm, const void* Cm, const float* Dskip,
                const void* z, const float* h0,
                void* y, float* h_final,
                void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ssm_ssd_fwd";
    if (B < 1 || H < 1 || P < 1 || N < 1 || L < 0 || chunk < 0)
        return fail(SSM_ERR_INVALID_ARG, fn, "B, H, P, N must be >= 1, L >= 0, chunk >= 0");
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, fn, "io must be SSM_F32 or SSM_BF16");
    const int Q = ssd_chunk(chunk);
    const char* why = ssm::ssd_unsupported_reason(L, H, P, N, Q, io == SSM_BF16);
    if (why[0] != '\0') return fail(SSM_ERR_UNSUPPORTED, fn, why);
    if (B > 65535) return fail(SSM_ERR_UNSUPPORTED, fn, "B must be <= 65535");
    if ((long long)B * H > (1LL << 24)) return fail(SSM_ERR_UNSUPPORTED, fn, "B * H must be <= 2^24");
    if (!product_ok({B, L, H, P}, 1LL << 40) || !product_ok({B, H, N, P}, 1LL << 40))
        return fail(SSM_ERR_INVALID_ARG, fn, "tensor sizes overflow");
    if (!A) return fail(SSM_ERR_INVALID_ARG, fn, "A is NULL");
    if (L > 0 && (!x || !delta || !Bm || !Cm || !y))
        return fail(SSM_ERR_INVALID_ARG, fn, "x, delta, Bm, Cm and y are required");
    const void* ptrs[] = {x, delta, A, Bm, Cm, Dskip, z, h0, y, h_final, workspace};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SSM_ERR_INVALID_ARG, fn, "every pointer must be 16-byte aligned");
    const size_t need = ssm::ssd_workspace_bytes(B, L, H, P, N, Q);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(SSM_ERR_WORKSPACE, fn, "workspace missing or smaller than ssm_ssd_workspace_size()");
    ssm::SsdArgs a{B, L, H, P, N, Q, io == SSM_BF16, x, delta, A, Bm, Cm, Dskip, z, h0, y, h_final, workspace};
    return hip_status(ssm::launch_ssd_fwd(a, static_cast<hipStream_t>(stream)), fn);
}

// ------------------------------------------------------------------ step
int ssm_step(int B, int D, int N, ssm_dtype_t io,
             float* state, const void* x, const void* delta, const float* A,
             const void* Bm, const void* Cm, const float* Dskip, const void* z,
             void* y, void* stream) {
    return step_impl("ssm_step", B, D, N, io, SSM_DISC_EULER, nullptr, 0, state, x, delta, A, Bm, Cm, Dskip, z,
                     y, stream);
}

int ssm_step_ex(int B, int D, int N, ssm_dtype_t io, ssm_disc_t disc,
                const float* delta_bias, int delta_softplus,
                float* state, const void* x, const void* delta, const float* A,
                const void* Bm, const void* Cm, const float* Dskip, const void* z,
                void* y, void* stream) {
    return step_impl("ssm_step_ex", B, D, N, io, disc, delta_bias, delta_softplus, state, x, delta, A, Bm, Cm,
                     Dskip, z, y, stream);
}

// ------------------------------------------------------------------ SSD step
int ssm_ssd_step(int B, int H, int P, int N, ssm_dtype_t io,
                 float* state, const void* x, const void* delta, const float* A,
                 const void* Bm, const void* Cm, const float* Dskip, const void* z,
                 void* y, void* stream) {
    const char* fn = "ssm_ssd_step";
    if (B < 1 || H < 1 || P < 1 || N < 1) return fail(SSM_ERR_INVALID_ARG, fn, "B, H, P, N must be >= 1");
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_INVALID_ARG, fn, "io must be SSM_F32 or SSM_BF16");
    if (!ssm::ssd_step_supported(P, N))
        return fail(SSM_ERR_UNSUPPORTED, fn, "P must be 64 and N one of 16, 32, 64, 128, 256");
    if ((long long)B * H > 0x7fffffffLL) return fail(SSM_ERR_UNSUPPORTED, fn, "B * H must be < 2^31");
    if (!product_ok({B, H, N, P}, 1LL << 40)) return fail(SSM_ERR_INVALID_ARG, fn, "tensor sizes overflow");
    if (!state || !x || !delta || !A || !Bm || !Cm || !y)
        return fail(SSM_ERR_INVALID_ARG, fn, "state, x, delta, A, Bm, Cm and y are required");
    const void* ptrs[] = {state, x, delta, A, Bm, Cm, Dskip, z, y};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SSM_ERR_INVALID_ARG, fn, "every pointer must be 16-byte aligned");
    ssm::SsdStepArgs a{B, H, P, N, io == SSM_BF16, state, x, delta, A, Bm, Cm, Dskip, z, y};
    return hip_status(ssm::launch_ssd_step(a, static_cast<hipStream_t>(stream)), fn);
}

// ------------------------------------------------------------------ diagnostics
int ssm_diag_valu_rate(int mode, int blocks, int iters, float* out, void* stream) {
    const char* fn = "ssm_diag_valu_rate";
    if (mode < 0 || mode > 4) return fail(SSM_ERR_INVALID_ARG, fn, "mode must be 0 .. 4");
    if (blocks < 1 || blocks > (1 << 20) || iters < 0) return fail(SSM_ERR_INVALID_ARG, fn, "bad blocks or iters");
    if (!out || !aligned16(out)) return fail(SSM_ERR_INVALID_ARG, fn, "out is NULL or not 16-byte aligned");
    return hip_status(ssm::launch_valu_rate(mode, blocks, iters, out, static_cast<hipStream_t>(stream)), fn);
}

int ssm_diag_stream_scale(float* p, size_t n, float s, void* stream) {
    const char* fn = "ssm_diag_stream_scale";
    if (!p || !aligned16(p) || n % 4 != 0 || n == 0)
        return fail(SSM_ERR_INVALID_ARG, fn, "p must be 16-byte aligned and n a positive multiple of 4");
    return hip_status(ssm::launch_stream_scale(p, n, s, static_cast<hipStream_t>(stream)), fn);
}

int ssm_diag_copy(const float* src, float* dst, size_t n, void* stream) {
    const char* fn = "ssm_diag_copy";
    if (!src || !dst || !aligned16(src) || !aligned16(dst) || n % 4 != 0 || n == 0)
        return fail(SSM_ERR_INVALID_ARG, fn, "pointers must be 16-byte aligned and n a positive multiple of 4");
    return hip_status(ssm::launch_copy(src, dst, n, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
