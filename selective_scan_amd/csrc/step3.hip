// Mamba-3 one-token decode step on gfx950 ("Efficient Sequence Modeling: From S4
// to Mamba-3", section 03 System, mamba3_minimal.py: the incremental form of the
// complex, exponential-trapezoidal recurrence). For each (batch, channel) and
// state n, in place:
//   alpha = exp(Delta (Are + i theta))
//   h     = alpha (h + (1 - lam) Delta B_prev[n] x_prev) + lam Delta B[n] x
//   y     = (sum_n C[n] Re h[n] + D x) silu(z)
// (x_prev, B_prev) is the previous token, the same pair ssm_scan3_fwd takes to
// continue a sequence; without it the previous token's term is zero.
//
// Bandwidth-bound: the complex state is read and written once. Lane layout: each
// lane owns two consecutive complex states of one channel (one 16-byte load and
// store of the state, 8-byte loads of Are and theta), so N/2 consecutive lanes
// share a channel and every state load or store instruction of a wave covers 1 KiB
// of contiguous state. C . Re h is summed over the channel's lanes with cross-lane
// shuffles; the channel's first lane writes y. Every load of a lane is issued before
// its state store (a load issued after a store would also wait for that store).
#include "common.h"
#include "step3.h"

namespace ssm {
namespace {

constexpr float kInv2Pi3 = 0.15915494309189535f;

template <bool BF16>
__device__ __forceinline__ float ld1(const void* p, size_t i) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}

// elements i and i + 1 of an io tensor (i even)
template <bool BF16>
__device__ __forceinline__ float2 ld2(const void* p, size_t i) {
    if constexpr (BF16) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
        return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
    } else {
        return *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i);
    }
}

// LPC: lanes per channel (N / 2), a power of two <= 64
template <bool BF16, int LPC>
__global__ void __launch_bounds__(256) step3_kernel(Step3Args a) {
    const size_t total = (size_t)a.B * a.D * LPC;
    const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = gid < total;
    const size_t g = live ? gid : total - 1;  // lanes past the end recompute the last pair and store nothing
    const size_t ch = g / LPC;                 // (batch, channel)
    const int j = (int)(g % LPC);              // pair index within the channel
    const int b = (int)(ch / a.D), d = (int)(ch % a.D);
    const int N = 2 * LPC, n0 = 2 * j;

    float4* sp = reinterpret_cast<float4*>(a.state) + g;  // states n0, n0 + 1 as (re, im, re, im)
    const float4 h = *sp;
    const float2 Ar = *reinterpret_cast<const float2*>(a.Are + (size_t)d * N + n0);
    const float2 Th = *reinterpret_cast<const float2*>(a.theta + (size_t)d * N + n0);
    const float2 Bv = ld2<BF16>(a.Bm, (size_t)b * N + n0);
    const float2 Cv = ld2<BF16>(a.Cm, (size_t)b * N + n0);
    const bool prev = a.x_prev != nullptr;
    const float2 Bp = prev ? ld2<BF16>(a.B_prev, (size_t)b * N + n0) : make_float2(0.0f, 0.0f);
    const float xp = prev ? ld1<BF16>(a.x_prev, ch) : 0.0f;
    const float xv = ld1<BF16>(a.x, ch), dv = ld1<BF16>(a.delta, ch), lv = ld1<BF16>(a.lam, ch);
    const float zv = a.z != nullptr ? ld1<BF16>(a.z, ch) : 0.0f;
    const float Dv = a.Dskip != nullptr ? a.Dskip[d] : 0.0f;

    const float q = (1.0f - lv) * dv * xp;  // weight of B_prev[n] (times alpha)
    const float r = lv * dv * xv;           // weight of B[n]
    float4 o;
    float yp;
    {
        const float m = exp2_fast(dv * Ar.x * kLog2e), ph = dv * Th.x * kInv2Pi3;
        const float ar = m * __builtin_amdgcn_cosf(ph), ai = m * __builtin_amdgcn_sinf(ph);
        const float gr = __builtin_fmaf(q, Bp.x, h.x);
        o.x = __builtin_fmaf(ar, gr, __builtin_fmaf(-ai, h.y, r * Bv.x));
        o.y = __builtin_fmaf(ai, gr, ar * h.y);
    }
    {
        const float m = exp2_fast(dv * Ar.y * kLog2e), ph = dv * Th.y * kInv2Pi3;
        const float ar = m * __builtin_amdgcn_cosf(ph), ai = m * __builtin_amdgcn_sinf(ph);
        const float gr = __builtin_fmaf(q, Bp.y, h.z);
        o.z = __builtin_fmaf(ar, gr, __builtin_fmaf(-ai, h.w, r * Bv.y));
        o.w = __builtin_fmaf(ai, gr, ar * h.w);
    }
    yp = __builtin_fmaf(Cv.x, o.x, Cv.y * o.z);
    // sum over the channel's LPC lanes (aligned groups of consecutive lanes)
#pragma unroll
    for (int off = 1; off < LPC; off <<= 1) yp += __shfl_xor(yp, off, 64);
    if (live) *sp = o;
    if (live && j == 0) {
        float v = __builtin_fmaf(Dv, xv, yp);
        if (a.z != nullptr) v *= silu(zv);
        if constexpr (BF16) static_cast<uint16_t*>(a.y)[ch] = f32_to_bf16(v);
        else static_cast<float*>(a.y)[ch] = v;
    }
}

template <bool BF16>
hipError_t launch_t(const Step3Args& a, hipStream_t st) {
    const size_t lanes = (size_t)a.B * a.D * (a.N / 2);
    const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
    switch (a.N) {
        case 4: launch((step3_kernel<BF16, 2>), grid, block, 0, st, a); break;
        case 8: launch((step3_kernel<BF16, 4>), grid, block, 0, st, a); break;
        case 16: launch((step3_kernel<BF16, 8>), grid, block, 0, st, a); break;
        case 32: launch((step3_kernel<BF16, 16>), grid, block, 0, st, a); break;
        case 64: launch((step3_kernel<BF16, 32>), grid, block, 0, st, a); break;
        case 128: launch((step3_kernel<BF16, 64>), grid, block, 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool step3_supported_n(int N) { return N == 4 || N == 8 || N == 16 || N == 32 || N == 64 || N == 128; }

hipError_t launch_step3(const Step3Args& a, hipStream_t st) {
    return a.bf16 ? launch_t<true>(a, st) : launch_t<false>(a, st);
}

}  // namespace ssm
