// One-token recurrent decode step on gfx950, state updated in place:
//   h = exp(Delta A) h + Delta B x,  y = (C . h + D x) silu(z)
// ("Efficient Sequence Modeling: From S4 to Mamba-3", section 03: mamba_minimal.py
// has an incremental step() for decoding; section 09: step() equals a full forward).
//
// Bandwidth-bound: the state row of a (batch, channel) pair is N contiguous floats,
// and A is [D][N], so both are walked as flat float4 arrays. QPC = N/4 consecutive
// lanes share a channel, each owning one float4 quarter of its state, so every
// load/store instruction of a wave covers 1 KiB of contiguous state. Each lane
// handles kReps quarters spaced one workgroup apart; the quarter index within the
// channel is the same for all of them (the workgroup size is a multiple of QPC),
// so a lane reads its 4 B and 4 C values once. C . h is summed over the QPC lanes
// with cross-lane shuffles and the channel's first lane writes y.
#include "common.h"
#include "launch.h"

#ifndef SSM_STEP_REPS
#define SSM_STEP_REPS 2
#endif
#ifndef SSM_STEP_THREADS
#define SSM_STEP_THREADS 256
#endif

namespace ssm {
namespace {

constexpr int kStepThreads = SSM_STEP_THREADS;
constexpr int kReps = SSM_STEP_REPS;

template <bool BF16>
__device__ __forceinline__ float load_io_at(const void* p, size_t i) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}

// The 4 values of row `row` of an [.][N] io-dtype matrix starting at column 4q.
template <int N, bool BF16>
__device__ __forceinline__ float4 load_quarter(const void* p, int row, int q) {
    if constexpr (BF16) {
        const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + (size_t)row * N + 4 * q);
        return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    } else {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + (size_t)row * N + 4 * q);
    }
}

template <int N, bool BF16, bool HAS_Z, bool HAS_D>
__global__ void __launch_bounds__(kStepThreads) step_kernel(StepArgs a) {
    constexpr int QPC = N / 4;
    static_assert(kStepThreads % QPC == 0, "a channel's lanes must not straddle two reps");
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int q = t & (QPC - 1);
    const int D = a.D;
    const int F = D * QPC;  // float4 quarters in one batch row
    const int f0 = blockIdx.x * (kStepThreads * kReps) + t;

    const float4 Bq = load_quarter<N, BF16>(a.Bm, b, q);
    const float4 Cq = load_quarter<N, BF16>(a.Cm, b, q);
    float4* st = reinterpret_cast<float4*>(a.state + (size_t)b * D * N);
    const float4* Af = reinterpret_cast<const float4*>(a.A);

    // every load of both reps before any store (a load issued after a store would
    // also wait for that store) and without a branch (so none is waited for before
    // the next is issued): lanes past the row read its last quarter and store nothing
    float4 h[kReps], A4[kReps];
    float dv[kReps], xv[kReps], zv[kReps], dk[kReps];
#pragma unroll
    for (int r = 0; r < kReps; ++r) {
        const int fc = min(f0 + r * kStepThreads, F - 1);
        const int d = fc / QPC;
        h[r] = st[fc];
        A4[r] = Af[fc];
        dv[r] = load_io_at<BF16>(a.delta, (size_t)b * D + d);
        xv[r] = load_io_at<BF16>(a.x, (size_t)b * D + d);
        zv[r] = HAS_Z ? load_io_at<BF16>(a.z, (size_t)b * D + d) : 0.0f;
        dk[r] = HAS_D ? a.Dskip[d] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < kReps; ++r) {
        const int f = f0 + r * kStepThreads;
        const float dt = dv[r], u = dv[r] * xv[r];
        float4 hn;
        hn.x = __builtin_fmaf(exp2_fast(dt * kLog2e * A4[r].x), h[r].x, u * Bq.x);
        hn.y = __builtin_fmaf(exp2_fast(dt * kLog2e * A4[r].y), h[r].y, u * Bq.y);
        hn.z = __builtin_fmaf(exp2_fast(dt * kLog2e * A4[r].z), h[r].z, u * Bq.z);
        hn.w = __builtin_fmaf(exp2_fast(dt * kLog2e * A4[r].w), h[r].w, u * Bq.w);
        if (f < F) st[f] = hn;
        float p = __builtin_fmaf(Cq.x, hn.x, Cq.y * hn.y) + __builtin_fmaf(Cq.z, hn.z, Cq.w * hn.w);
#pragma unroll
        for (int o = QPC / 2; o >= 1; o >>= 1) p += __shfl_xor(p, o);
        if (q == 0 && f < F) {
            const int d = f / QPC;
            float v = p;
            if constexpr (HAS_D) v = __builtin_fmaf(dk[r], xv[r], v);
            if constexpr (HAS_Z) v *= silu(zv[r]);
            if constexpr (BF16) static_cast<uint16_t*>(a.y)[(size_t)b * D + d] = f32_to_bf16(v);
            else static_cast<float*>(a.y)[(size_t)b * D + d] = v;
        }
    }
}

// Discretisation variants of the step (bandwidth-bound, so the options are
// runtime flags): Delta = [softplus](delta + bias); exponential-Euler or the exact
// zero-order hold Bbar x = (e^z - 1)/A B x, z = Delta A, with the series
// Delta (1 + z/2 + z^2/6 + z^3/24) where |z| < 1/32 (truncation < 1e-8 relative).
__device__ __forceinline__ float step_softplus(float v) {
    const float e = exp2_fast(-fabsf(v) * kLog2e);
    const float series = e * __builtin_fmaf(e, __builtin_fmaf(e, 1.0f / 3.0f, -0.5f), 1.0f);
    const float lg = __builtin_amdgcn_logf(1.0f + e) * 0.69314718055994531f;
    return fmaxf(v, 0.0f) + (e < 0.015625f ? series : lg);
}

__device__ __forceinline__ float step_input(float ab, float hv, float dt, float A, float xb, bool zoh) {
    if (!zoh) return __builtin_fmaf(ab, hv, dt * xb);
    const float z = dt * A;
    const float taylor =
        dt * __builtin_fmaf(z, __builtin_fmaf(z, __builtin_fmaf(z, 1.0f / 24.0f, 1.0f / 6.0f), 0.5f), 1.0f);
    const float coef = fabsf(z) < 0.03125f ? taylor : (ab - 1.0f) / A;
    return __builtin_fmaf(ab, hv, coef * xb);
}

template <int N, bool BF16>
__global__ void __launch_bounds__(kStepThreads) step_kernel_var(StepArgs a) {
    constexpr int QPC = N / 4;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int q = t & (QPC - 1);
    const int D = a.D;
    const int F = D * QPC;
    const int f0 = blockIdx.x * (kStepThreads * kReps) + t;
    const bool zoh = a.disc == 1, sp = a.delta_softplus != 0;
    const float4 Bq = load_quarter<N, BF16>(a.Bm, b, q);
    const float4 Cq = load_quarter<N, BF16>(a.Cm, b, q);
    float4* st = reinterpret_cast<float4*>(a.state + (size_t)b * D * N);
    const float4* Af = reinterpret_cast<const float4*>(a.A);
    // every load of the lane is issued before its first state store (a load issued
    // after a store would also wait for the store) and without a branch (so none is
    // waited for before the next is issued): an absent bias, skip or gate reads a
    // tensor of the same shape instead and is not used; lanes past the row read its
    // last quarter and store nothing
    const float* biasp = a.delta_bias != nullptr ? a.delta_bias : a.A;
    const float* skp = a.Dskip != nullptr ? a.Dskip : a.A;
    const void* zp = a.z != nullptr ? a.z : a.x;
    float dl[kReps], bias[kReps], xs[kReps], zs[kReps], sk[kReps];
    float4 A4s[kReps], hs[kReps];
#pragma unroll
    for (int r = 0; r < kReps; ++r) {
        const int fc = min(f0 + r * kStepThreads, F - 1);
        const int d = fc / QPC;
        dl[r] = load_io_at<BF16>(a.delta, (size_t)b * D + d);
        bias[r] = biasp[d];
        xs[r] = load_io_at<BF16>(a.x, (size_t)b * D + d);
        zs[r] = load_io_at<BF16>(zp, (size_t)b * D + d);
        sk[r] = skp[d];
        A4s[r] = Af[fc];
        hs[r] = st[fc];
    }
#pragma unroll
    for (int r = 0; r < kReps; ++r) {
        const int f = f0 + r * kStepThreads;
        const int d = (f < F ? f : F - 1) / QPC;
        float dt = dl[r];
        if (a.delta_bias != nullptr) dt += bias[r];
        if (sp) dt = step_softplus(dt);
        const float xv = xs[r];
        const float4 A4 = A4s[r];
        const float4 h = hs[r];
        float4 hn;
        hn.x = step_input(exp2_fast(dt * kLog2e * A4.x), h.x, dt, A4.x, xv * Bq.x, zoh);
        hn.y = step_input(exp2_fast(dt * kLog2e * A4.y), h.y, dt, A4.y, xv * Bq.y, zoh);
        hn.z = step_input(exp2_fast(dt * kLog2e * A4.z), h.z, dt, A4.z, xv * Bq.z, zoh);
        hn.w = step_input(exp2_fast(dt * kLog2e * A4.w), h.w, dt, A4.w, xv * Bq.w, zoh);
        if (f < F) st[f] = hn;
        float p = __builtin_fmaf(Cq.x, hn.x, Cq.y * hn.y) + __builtin_fmaf(Cq.z, hn.z, Cq.w * hn.w);
#pragma unroll
        for (int o = QPC / 2; o >= 1; o >>= 1) p += __shfl_xor(p, o);
        if (q == 0 && f < F) {
            float v = p;
            if (a.Dskip != nullptr) v = __builtin_fmaf(sk[r], xv, v);
            if (a.z != nullptr) v *= silu(zs[r]);
            if constexpr (BF16) static_cast<uint16_t*>(a.y)[(size_t)b * D + d] = f32_to_bf16(v);
            else static_cast<float*>(a.y)[(size_t)b * D + d] = v;
        }
    }
}

template <int N, bool BF16>
hipError_t launch_n(const StepArgs& a, hipStream_t st) {
    const long F = (long)a.D * (N / 4);
    const dim3 grid((unsigned)((F + kStepThreads * kReps - 1) / (kStepThreads * kReps)), (unsigned)a.B);
    const bool hz = a.z != nullptr, hd = a.Dskip != nullptr;
    if (hz && hd) launch((step_kernel<N, BF16, true, true>), grid, dim3(kStepThreads), 0, st, a);
    else if (hz) launch((step_kernel<N, BF16, true, false>), grid, dim3(kStepThreads), 0, st, a);
    else if (hd) launch((step_kernel<N, BF16, false, true>), grid, dim3(kStepThreads), 0, st, a);
    else launch((step_kernel<N, BF16, false, false>), grid, dim3(kStepThreads), 0, st, a);
    return hipGetLastError();
}

template <int N, bool BF16>
hipError_t launch_var_n(const StepArgs& a, hipStream_t st) {
    const long F = (long)a.D * (N / 4);
    const dim3 grid((unsigned)((F + kStepThreads * kReps - 1) / (kStepThreads * kReps)), (unsigned)a.B);
    launch((step_kernel_var<N, BF16>), grid, dim3(kStepThreads), 0, st, a);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_var_dtype(const StepArgs& a, hipStream_t st) {
    switch (a.N) {
        case 4: return launch_var_n<4, BF16>(a, st);
        case 8: return launch_var_n<8, BF16>(a, st);
        case 16: return launch_var_n<16, BF16>(a, st);
        case 32: return launch_var_n<32, BF16>(a, st);
        case 64: return launch_var_n<64, BF16>(a, st);
        case 128: return launch_var_n<128, BF16>(a, st);
        case 256: return launch_var_n<256, BF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
hipError_t launch_dtype(const StepArgs& a, hipStream_t st) {
    switch (a.N) {
        case 4: return launch_n<4, BF16>(a, st);
        case 8: return launch_n<8, BF16>(a, st);
        case 16: return launch_n<16, BF16>(a, st);
        case 32: return launch_n<32, BF16>(a, st);
        case 64: return launch_n<64, BF16>(a, st);
        case 128: return launch_n<128, BF16>(a, st);
        case 256: return launch_n<256, BF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool step_supported_n(int N) {
    return N == 4 || N == 8 || N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
}

hipError_t launch_step(const StepArgs& a, hipStream_t st) {
    return a.bf16 ? launch_dtype<true>(a, st) : launch_dtype<false>(a, st);
}

hipError_t launch_step_var(const StepArgs& a, hipStream_t st) {
    return a.bf16 ? launch_var_dtype<true>(a, st) : launch_var_dtype<false>(a, st);
}

}  // namespace ssm
