// One-token decode step of the Mamba-2 form on gfx950, state updated in place
// ("Efficient Sequence Modeling: From S4 to Mamba-3", section 03: the
// incremental step() of mamba_minimal.py, here with mamba2_minimal.py's scalar
// decay per head and (N, P) state per head):
//   a = exp(Delta A_h),  S[n, p] = a S[n, p] + Delta B[n] x[p],
//   y[p] = (sum_n C[n] S[n, p] + D_h x[p]) silu(z[p])
//
// Bandwidth-bound: one workgroup of 256 lanes per (batch, head). Lane
// (ng = lane / 16, pq = lane % 16) owns the float4 S[n, 4pq .. 4pq+3] of the
// rows n = ng, ng + 16, ... ; all of them are loaded before any is used, so a
// wave has N/16 16-byte loads in flight, and every load/store instruction of a
// wave covers four rows of 256 contiguous bytes. y is summed over the 16
// row groups: within a wave across lanes 16 and 32 apart, then across the four
// waves through LDS.
#include "common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kSP = 64;        // head dim P handled
constexpr int kSThreads = 256;

template <bool BF16>
__device__ __forceinline__ float ld1(const void* p, size_t i) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}

// four consecutive io values starting at element i (i a multiple of 4)
template <bool BF16>
__device__ __forceinline__ float4 ld4(const void* p, size_t i) {
    if constexpr (BF16) {
        const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    } else {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    }
}

template <bool BF16>
__device__ __forceinline__ void st4(void* p, size_t i, float4 v) {
    if constexpr (BF16) {
        uint2 w;
        w.x = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
        w.y = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = w;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = v;
    }
}

template <int N, bool BF16, bool HAS_Z, bool HAS_D>
__global__ void __launch_bounds__(kSThreads) ssd_step_kernel(SsdStepArgs a) {
    constexpr int R = N / 16;  // rows per lane
    __shared__ float4 red[kSThreads / 64][16];
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, pq = tid & 15, ng = tid >> 4;
    float4* S = reinterpret_cast<float4*>(a.state + (size_t)bh * N * kSP) + pq;

    // Every load is issued before the first state store: stores count against the
    // same outstanding-memory counter as loads, so a load issued after a store would
    // also wait for that store.
    float4 s[R];
    float bn[R], cn[R];
#pragma unroll
    for (int k = 0; k < R; ++k) s[k] = S[(ng + 16 * k) * (kSP / 4)];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        bn[k] = ld1<BF16>(a.Bm, (size_t)b * N + ng + 16 * k);
        cn[k] = ld1<BF16>(a.Cm, (size_t)b * N + ng + 16 * k);
    }
    const float dt = ld1<BF16>(a.delta, bh);
    const float Ah = a.A[h];
    const float4 xv = ld4<BF16>(a.x, (size_t)bh * kSP + 4 * pq);
    const float dh = HAS_D ? a.Dskip[h] : 0.0f;
    const float4 zv = HAS_Z ? ld4<BF16>(a.z, (size_t)bh * kSP + 4 * pq) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float decay = exp2_fast(dt * Ah * kLog2e);
    const float4 u = make_float4(dt * xv.x, dt * xv.y, dt * xv.z, dt * xv.w);
    float4 yp = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int n = ng + 16 * k;
        float4 v;
        v.x = __builtin_fmaf(decay, s[k].x, bn[k] * u.x);
        v.y = __builtin_fmaf(decay, s[k].y, bn[k] * u.y);
        v.z = __builtin_fmaf(decay, s[k].z, bn[k] * u.z);
        v.w = __builtin_fmaf(decay, s[k].w, bn[k] * u.w);
        S[n * (kSP / 4)] = v;
        yp.x = __builtin_fmaf(cn[k], v.x, yp.x);
        yp.y = __builtin_fmaf(cn[k], v.y, yp.y);
        yp.z = __builtin_fmaf(cn[k], v.z, yp.z);
        yp.w = __builtin_fmaf(cn[k], v.w, yp.w);
    }
    // sum over the 4 row groups of this wave (lanes 16 and 32 apart) ...
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
        yp.x += __shfl_xor(yp.x, o);
        yp.y += __shfl_xor(yp.y, o);
        yp.z += __shfl_xor(yp.z, o);
        yp.w += __shfl_xor(yp.w, o);
    }
    // ... then over the 4 waves
    if ((tid & 63) < 16) red[tid >> 6][pq] = yp;
    __syncthreads();
    if (tid < 16) {
        float4 v = red[0][pq];
#pragma unroll
        for (int w = 1; w < kSThreads / 64; ++w) {
            v.x += red[w][pq].x;
            v.y += red[w][pq].y;
            v.z += red[w][pq].z;
            v.w += red[w][pq].w;
        }
        if constexpr (HAS_D) {
            v.x = __builtin_fmaf(dh, xv.x, v.x);
            v.y = __builtin_fmaf(dh, xv.y, v.y);
            v.z = __builtin_fmaf(dh, xv.z, v.z);
            v.w = __builtin_fmaf(dh, xv.w, v.w);
        }
        if constexpr (HAS_Z) {
            v.x *= silu(zv.x);
            v.y *= silu(zv.y);
            v.z *= silu(zv.z);
            v.w *= silu(zv.w);
        }
        st4<BF16>(a.y, (size_t)bh * kSP + 4 * pq, v);
    }
}

template <int N, bool BF16>
hipError_t launch_n(const SsdStepArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((long)a.B * a.H));
    const bool hz = a.z != nullptr, hd = a.Dskip != nullptr;
    if (hz && hd) launch((ssd_step_kernel<N, BF16, true, true>), grid, dim3(kSThreads), 0, st, a);
    else if (hz) launch((ssd_step_kernel<N, BF16, true, false>), grid, dim3(kSThreads), 0, st, a);
    else if (hd) launch((ssd_step_kernel<N, BF16, false, true>), grid, dim3(kSThreads), 0, st, a);
    else launch((ssd_step_kernel<N, BF16, false, false>), grid, dim3(kSThreads), 0, st, a);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const SsdStepArgs& a, hipStream_t st) {
    switch (a.N) {
        case 16: return launch_n<16, BF16>(a, st);
        case 32: return launch_n<32, BF16>(a, st);
        case 64: return launch_n<64, BF16>(a, st);
        case 128: return launch_n<128, BF16>(a, st);
        case 256: return launch_n<256, BF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool ssd_step_supported(int P, int N) {
    return P == kSP && (N == 16 || N == 32 || N == 64 || N == 128 || N == 256);
}

hipError_t launch_ssd_step(const SsdStepArgs& a, hipStream_t st) {
    return a.bf16 ? launch_dtype<true>(a, st) : launch_dtype<false>(a, st);
}

}  // namespace ssm
