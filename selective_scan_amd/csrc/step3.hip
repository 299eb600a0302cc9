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
// Bandwidth-bound: the complex state is read and written once. Lane layout: a lane
// owns two consecutive complex states of one channel (one 16-byte load and store of
// the state, 8-byte loads of Are and theta) in each of kReps3 channels a workgroup
// apart, so N/2 consecutive lanes share a channel and every state load or store
// instruction of a wave covers 1 KiB of contiguous state. C . Re h is summed over
// the channel's lanes with cross-lane shuffles; the channel's first lane writes y.
// Every load of a lane is issued before its first state store (a load issued after
// a store would also wait for that store).
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

#ifndef SSM_STEP3_THREADS
#define SSM_STEP3_THREADS 256
#endif
#ifndef SSM_STEP3_REPS
#define SSM_STEP3_REPS 4
#endif
constexpr int kThreads3 = SSM_STEP3_THREADS;
// pairs per lane, one workgroup's width apart: at B64 D3072 N16, 4 pairs took a
// step from 13.7 (1 pair) and 13.0 (2) to 11.6 us with the state MALL-resident and
// from 16.3 to 15.5 us cold; 8 pairs were slower again (13.7, 17.8 us), and 64-,
// 128- and 512-lane workgroups were within 0.5 us of 256
constexpr int kReps3 = SSM_STEP3_REPS;

// LPC: lanes per channel (N / 2), a power of two <= 64. Workgroup (x, batch row b)
// covers kThreads3 * kReps3 consecutive pairs of row b; a lane's pairs are
// kThreads3 apart, so they share the pair index j within their channels and the
// lane reads its B, C and B_prev values once.
template <bool BF16, int LPC>
__global__ void __launch_bounds__(kThreads3) step3_kernel(Step3Args a) {
    constexpr int N = 2 * LPC;
    static_assert(kThreads3 % LPC == 0, "a channel's lanes must not straddle two reps");
    const int b = blockIdx.y, t = threadIdx.x;
    const int j = t & (LPC - 1), n0 = 2 * j;
    const int F = a.D * LPC;  // pairs in one batch row
    const int f0 = blockIdx.x * (kThreads3 * kReps3) + t;
    const bool prev = a.x_prev != nullptr, hz = a.z != nullptr, hd = a.Dskip != nullptr;

    const float2 Bv = ld2<BF16>(a.Bm, (size_t)b * N + n0);
    const float2 Cv = ld2<BF16>(a.Cm, (size_t)b * N + n0);
    const float2 Bp = prev ? ld2<BF16>(a.B_prev, (size_t)b * N + n0) : make_float2(0.0f, 0.0f);
    float4* sp = reinterpret_cast<float4*>(a.state) + (size_t)b * F;
    // every load of all the lane's pairs before the first store; pairs past the row read the
    // row's last pair and store nothing
    float4 h[kReps3];
    float2 Ar[kReps3], Th[kReps3];
    float xv[kReps3], dv[kReps3], lv[kReps3], zv[kReps3], xp[kReps3], Dv[kReps3];
#pragma unroll
    for (int r = 0; r < kReps3; ++r) {
        const int f = min(f0 + r * kThreads3, F - 1);
        const int d = f / LPC;
        const size_t ch = (size_t)b * a.D + d;
        h[r] = sp[f];
        Ar[r] = *reinterpret_cast<const float2*>(a.Are + (size_t)d * N + n0);
        Th[r] = *reinterpret_cast<const float2*>(a.theta + (size_t)d * N + n0);
        xv[r] = ld1<BF16>(a.x, ch);
        dv[r] = ld1<BF16>(a.delta, ch);
        lv[r] = ld1<BF16>(a.lam, ch);
        zv[r] = hz ? ld1<BF16>(a.z, ch) : 0.0f;
        xp[r] = prev ? ld1<BF16>(a.x_prev, ch) : 0.0f;
        Dv[r] = hd ? a.Dskip[d] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < kReps3; ++r) {
        const int f = f0 + r * kThreads3;
        const float q = (1.0f - lv[r]) * dv[r] * xp[r];  // weight of B_prev[n] (times alpha)
        const float rr = lv[r] * dv[r] * xv[r];         // weight of B[n]
        float4 o;
        {
            const float m = exp2_fast(dv[r] * Ar[r].x * kLog2e), ph = dv[r] * Th[r].x * kInv2Pi3;
            const float ar = m * __builtin_amdgcn_cosf(ph), ai = m * __builtin_amdgcn_sinf(ph);
            const float gr = __builtin_fmaf(q, Bp.x, h[r].x);
            o.x = __builtin_fmaf(ar, gr, __builtin_fmaf(-ai, h[r].y, rr * Bv.x));
            o.y = __builtin_fmaf(ai, gr, ar * h[r].y);
        }
        {
            const float m = exp2_fast(dv[r] * Ar[r].y * kLog2e), ph = dv[r] * Th[r].y * kInv2Pi3;
            const float ar = m * __builtin_amdgcn_cosf(ph), ai = m * __builtin_amdgcn_sinf(ph);
            const float gr = __builtin_fmaf(q, Bp.y, h[r].z);
            o.z = __builtin_fmaf(ar, gr, __builtin_fmaf(-ai, h[r].w, rr * Bv.y));
            o.w = __builtin_fmaf(ai, gr, ar * h[r].w);
        }
        float yp = __builtin_fmaf(Cv.x, o.x, Cv.y * o.z);
        // sum over the channel's LPC lanes (aligned groups of consecutive lanes)
#pragma unroll
        for (int off = 1; off < LPC; off <<= 1) yp += __shfl_xor(yp, off, 64);
        if (f < F) {
            sp[f] = o;
            if (j == 0) {
                float v = __builtin_fmaf(Dv[r], xv[r], yp);
                if (hz) v *= silu(zv[r]);
                const size_t ch = (size_t)b * a.D + f / LPC;
                if constexpr (BF16) static_cast<uint16_t*>(a.y)[ch] = f32_to_bf16(v);
                else static_cast<float*>(a.y)[ch] = v;
            }
        }
    }
}

template <bool BF16>
hipError_t launch_t(const Step3Args& a, hipStream_t st) {
    const long F = (long)a.D * (a.N / 2);
    const dim3 grid((unsigned)((F + kThreads3 * kReps3 - 1) / (kThreads3 * kReps3)), (unsigned)a.B), block(kThreads3);
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
