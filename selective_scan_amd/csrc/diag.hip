// Diagnostic kernels for the benchmark (not part of the scan itself):
//  - VALU issue-rate probes: long chains of v_exp_f32 only, of v_fma_f32 only, of
//    one v_exp_f32 per three v_fma_f32, of v_sin_f32 only and of v_cos_f32 only, so
//    the bench can measure what the transcendental unit costs relative to an FMA on
//    the chip it runs on;
//  - an in-place scale of an fp32 array, the pure-streaming floor a decode step
//    (read the state, write it back) is compared with;
//  - a plain device copy, the reference that scales the HBM byte counters and the
//    copy bandwidth the bench reports as context.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "extras.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kChains = 8;  // independent dependency chains per lane

// MODE 0: exp only, 1: fma only, 2: one exp per three fma, 3: v_sin_f32 only,
// 4: v_cos_f32 only. Modes 0-2 keep every chain in [0.5, 1] (2^-x of x in [0.5, 1];
// the fma contracts towards 0.75), modes 3 and 4 in [-1, 1] (the argument is in
// revolutions), so no special value ever enters the pipes. `iters` rounds of
// kChains x 4 ops per lane.
template <int MODE>
__global__ void __launch_bounds__(256) valu_rate(float* out, int iters) {
    float v[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) v[c] = 0.5f + 0.01f * (float)((threadIdx.x + c) & 31);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                if constexpr (MODE == 0) {
                    v[c] = __builtin_amdgcn_exp2f(-v[c]);
                } else if constexpr (MODE == 1) {
                    v[c] = __builtin_fmaf(v[c], 0.5f, 0.375f);
                } else if constexpr (MODE == 3) {
                    v[c] = __builtin_amdgcn_sinf(v[c]);
                } else if constexpr (MODE == 4) {
                    v[c] = __builtin_amdgcn_cosf(v[c]);
                } else {
                    if (r == 3) v[c] = __builtin_amdgcn_exp2f(-v[c]);
                    else v[c] = __builtin_fmaf(v[c], 0.5f, 0.375f);
                }
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += v[c];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// p[i] *= s over n floats; each lane issues all of its 16-byte loads before its
// first store (loads issued after a store would also wait for that store).
constexpr int kScaleVec = 4;  // float4 per lane per launch round
__global__ void __launch_bounds__(256) stream_scale(float4* __restrict__ p, size_t n4, float s) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i < n4; i += stride * kScaleVec) {
        float4 v[kScaleVec];
#pragma unroll
        for (int k = 0; k < kScaleVec; ++k) {
            const size_t j = i + k * stride;
            v[k] = p[j < n4 ? j : i];
        }
#pragma unroll
        for (int k = 0; k < kScaleVec; ++k) {
            const size_t j = i + k * stride;
            if (j < n4) p[j] = make_float4(v[k].x * s, v[k].y * s, v[k].z * s, v[k].w * s);
        }
    }
}

// dst = src over n4 float4; like stream_scale, each lane issues kScaleVec loads
// before its first store
__global__ void __launch_bounds__(256) copy16(const float4* __restrict__ src, float4* __restrict__ dst, size_t n4) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride * kScaleVec) {
        float4 v[kScaleVec];
#pragma unroll
        for (int k = 0; k < kScaleVec; ++k) {
            const size_t j = i + k * stride;
            v[k] = src[j < n4 ? j : i];
        }
#pragma unroll
        for (int k = 0; k < kScaleVec; ++k) {
            const size_t j = i + k * stride;
            if (j < n4) dst[j] = v[k];
        }
    }
}

}  // namespace

hipError_t launch_valu_rate(int mode, int blocks, int iters, float* out, hipStream_t st) {
    const dim3 g(blocks), b(256);
    if (mode == 0) launch(valu_rate<0>, g, b, 0, st, out, iters);
    else if (mode == 1) launch(valu_rate<1>, g, b, 0, st, out, iters);
    else if (mode == 2) launch(valu_rate<2>, g, b, 0, st, out, iters);
    else if (mode == 3) launch(valu_rate<3>, g, b, 0, st, out, iters);
    else launch(valu_rate<4>, g, b, 0, st, out, iters);
    return hipGetLastError();
}

hipError_t launch_stream_scale(float* p, size_t n, float s, hipStream_t st) {
    const size_t n4 = n / 4;
    // one float4 per lane per round, kScaleVec rounds in flight per lane
    const size_t lanes = (n4 + kScaleVec - 1) / kScaleVec;
    const unsigned blocks = (unsigned)std::max<size_t>(1, std::min<size_t>((lanes + 255) / 256, 1u << 20));
    launch(stream_scale, dim3(blocks), dim3(256), 0, st, reinterpret_cast<float4*>(p), n4, s);
    return hipGetLastError();
}

hipError_t launch_copy(const float* src, float* dst, size_t n, hipStream_t st) {
    const size_t n4 = n / 4;
    // one float4 per lane per round, kScaleVec rounds in flight per lane
    const size_t lanes = (n4 + kScaleVec - 1) / kScaleVec;
    const unsigned blocks = (unsigned)std::max<size_t>(1, std::min<size_t>((lanes + 255) / 256, 1u << 20));
    launch(copy16, dim3(blocks), dim3(256), 0, st, reinterpret_cast<const float4*>(src), reinterpret_cast<float4*>(dst),
           n4);
    return hipGetLastError();
}

}  // namespace ssm
