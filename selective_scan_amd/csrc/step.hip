// One-token recurrent decode step on gfx950, state updated in place:
//   h = exp(Delta A) h + Delta B x,  y = (C . h + D x) silu(z)
// ("Efficient Sequence Modeling: From S4 to Mamba-3", section 03: mamba_minimal.py
// has an incremental step() for decoding; section 09: step() equals a full forward).
//
// Bandwidth-bound: one lane per (batch, channel) reads its N-float state row and
// its A row with 16-byte vector loads, B and C of its batch row are wave-uniform
// (scalar loads), and the state is written back once. Workgroups never straddle
// two batch rows, so the uniform loads are valid for every lane.
#include "common.h"
#include "launch.h"

namespace ssm {
namespace {

template <int N, bool BF16, bool HAS_Z, bool HAS_D>
__global__ void __launch_bounds__(256) step_kernel(StepArgs a) {
    const int b = blockIdx.y;
    const int d = blockIdx.x * blockDim.x + threadIdx.x;
    const int D = a.D;
    if (d >= D) return;
    const size_t i = (size_t)b * D + d;
    float dv, xv, zv = 0.0f;
    if constexpr (BF16) {
        dv = bf16_to_f32(static_cast<const uint16_t*>(a.delta)[i]);
        xv = bf16_to_f32(static_cast<const uint16_t*>(a.x)[i]);
        if constexpr (HAS_Z) zv = bf16_to_f32(static_cast<const uint16_t*>(a.z)[i]);
    } else {
        dv = static_cast<const float*>(a.delta)[i];
        xv = static_cast<const float*>(a.x)[i];
        if constexpr (HAS_Z) zv = static_cast<const float*>(a.z)[i];
    }
    float Bt[N], Ct[N];
    load_uniform_row<N, BF16>(a.Bm, b, Bt);
    load_uniform_row<N, BF16>(a.Cm, b, Ct);

    float4* st = reinterpret_cast<float4*>(a.state + i * N);
    const float4* Ar = reinterpret_cast<const float4*>(a.A + (size_t)d * N);
    float h[N], A2[N];
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        const float4 s4 = st[k];
        const float4 a4 = Ar[k];
        h[4 * k] = s4.x; h[4 * k + 1] = s4.y; h[4 * k + 2] = s4.z; h[4 * k + 3] = s4.w;
        A2[4 * k] = a4.x * kLog2e; A2[4 * k + 1] = a4.y * kLog2e;
        A2[4 * k + 2] = a4.z * kLog2e; A2[4 * k + 3] = a4.w * kLog2e;
    }
    const float u = dv * xv;
    float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        h[n] = __builtin_fmaf(exp2_fast(dv * A2[n]), h[n], u * Bt[n]);
        if (n & 1) y1 = __builtin_fmaf(Ct[n], h[n], y1);
        else y0 = __builtin_fmaf(Ct[n], h[n], y0);
    }
#pragma unroll
    for (int k = 0; k < N / 4; ++k) st[k] = make_float4(h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]);
    float v = y0 + y1;
    if constexpr (HAS_D) v = __builtin_fmaf(a.Dskip[d], xv, v);
    if constexpr (HAS_Z) v *= silu(zv);
    if constexpr (BF16) static_cast<uint16_t*>(a.y)[i] = f32_to_bf16(v);
    else static_cast<float*>(a.y)[i] = v;
}

template <int N, bool BF16>
hipError_t launch_n(const StepArgs& a, hipStream_t st) {
    const int threads = a.D >= 256 ? 256 : ((a.D + 63) / 64) * 64;
    const dim3 grid((unsigned)((a.D + threads - 1) / threads), (unsigned)a.B);
    const bool hz = a.z != nullptr, hd = a.Dskip != nullptr;
    profile_mark(st);
    if (hz && hd) hipLaunchKernelGGL((step_kernel<N, BF16, true, true>), grid, dim3(threads), 0, st, a);
    else if (hz) hipLaunchKernelGGL((step_kernel<N, BF16, true, false>), grid, dim3(threads), 0, st, a);
    else if (hd) hipLaunchKernelGGL((step_kernel<N, BF16, false, true>), grid, dim3(threads), 0, st, a);
    else hipLaunchKernelGGL((step_kernel<N, BF16, false, false>), grid, dim3(threads), 0, st, a);
    profile_mark(st);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const StepArgs& a, hipStream_t st) {
    switch (a.N) {
        case 4: return launch_n<4, BF16>(a, st);
        case 8: return launch_n<8, BF16>(a, st);
        case 16: return launch_n<16, BF16>(a, st);
        case 32: return launch_n<32, BF16>(a, st);
        case 64: return launch_n<64, BF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool step_supported_n(int N) { return N == 4 || N == 8 || N == 16 || N == 32 || N == 64; }

hipError_t launch_step(const StepArgs& a, hipStream_t st) {
    return a.bf16 ? launch_dtype<true>(a, st) : launch_dtype<false>(a, st);
}

}  // namespace ssm
