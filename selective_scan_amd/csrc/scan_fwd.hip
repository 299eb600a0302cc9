// Mamba-1 selective scan on gfx950: h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t,
// y_t = (C_t . h_t + D x_t) silu(z_t)  (Gu & Dao 2023; exponential-Euler
// discretisation as named by "Efficient Sequence Modeling: From S4 to Mamba-3",
// sections 03 and 04).
//
// Work mapping. One lane owns one (batch, channel) and keeps its N state values
// and its row A[d, :] (pre-scaled by log2 e) in VGPRs. All lanes of a wave share
// the time step, so B_t and C_t are wave-uniform: they are read with scalar loads
// into SGPRs and feed the VALU directly. x, Delta, z, y are streamed with buffer
// loads/stores whose per-step offset lives in an SGPR (no VALU address math).
// Per state update the hot loop issues v_mul (Delta*A), v_exp_f32, v_mul (u*B),
// v_fma (state) and v_fma (C.h).
//
// L-parallelism. B*D channels alone cannot fill 256 CUs, so the sequence is cut
// into S segments and scanned in three launches:
//   1. segment_aggregate: every segment but the last runs the recurrence from a
//      zero state and stores its end state H_s and sum(Delta) of the segment;
//   2. carry_combine: per (b, n, d), h_in(s+1) = exp(A sum(Delta_s)) h_in(s) + H_s
//      sequentially over segments (tiny), written over H_s;
//   3. segment_final: every segment runs the recurrence again from its true
//      carried-in state and writes y (and h_final for the last segment).
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace ssm {
namespace {

constexpr int kPrefetch = 4;

struct Geom {
    int S, Ls;
    int threads;  // lanes per workgroup (multiple of 64, <= 256)
};

__host__ __device__ inline size_t ws_h_elems(int B, int S, int N, int D) {
    return (size_t)B * (S - 1) * N * D;
}

template <int N, bool BF16, bool FINAL, bool HAS_Z, bool HAS_D>
__global__ void __launch_bounds__(256)
segment_kernel(ScanArgs a, int S, int Ls) {
    constexpr uint32_t es = BF16 ? 2 : 4;
    const int seg = blockIdx.x;
    const int b = blockIdx.z;
    const int d = blockIdx.y * blockDim.x + threadIdx.x;
    const int D = a.D, L = a.L;
    const int dc = d < D ? d : D - 1;   // lanes past D mirror the last channel, never store
    const int t0 = seg * Ls;
    const int len = min(Ls, L - t0);
    const size_t row0 = (size_t)b * L + t0;  // first (b, t) row of this segment
    const uint32_t seg_bytes = (uint32_t)len * (uint32_t)D * es;

    const char* xb = static_cast<const char*>(a.x) + row0 * D * es;
    const char* db = static_cast<const char*>(a.delta) + row0 * D * es;
    const auto rx = make_rsrc(xb, seg_bytes);
    const auto rd = make_rsrc(db, seg_bytes);
    // z and y descriptors (unused when not FINAL / no gate: they then point at x)
    const auto rz = make_rsrc((FINAL && HAS_Z) ? static_cast<const char*>(a.z) + row0 * D * es : xb,
                              seg_bytes);
    const auto ry = make_rsrc(FINAL ? static_cast<const char*>(a.y) + row0 * D * es : xb, seg_bytes);
    const uint32_t voff = (uint32_t)dc * es;
    const uint32_t rstride = (uint32_t)D * es;

    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = a.A[(size_t)dc * N + n] * kLog2e;

    float* wsH = static_cast<float*>(a.ws);
    float* wsSd = wsH + ws_h_elems(a.B, S, N, D);
    if (FINAL && seg > 0) {
        const float* hin = wsH + (((size_t)b * (S - 1) + (seg - 1)) * N) * D + dc;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = hin[(size_t)n * D];
    } else if (FINAL && a.h0 != nullptr) {
        const float* hp = a.h0 + ((size_t)b * D + dc) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = hp[n];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = 0.0f;
    }
    float Dv = 0.0f;
    if constexpr (FINAL && HAS_D) Dv = a.Dskip[dc];

    const void* Bbase = static_cast<const char*>(a.Bm) + row0 * N * es;
    const void* Cbase = static_cast<const char*>(a.Cm) + row0 * N * es;

    // prefetch ring of kPrefetch steps (steps past the end re-read the last row)
    float dq[kPrefetch], xq[kPrefetch], zq[kPrefetch];
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
        const uint32_t so = (uint32_t)min(k, len - 1) * rstride;
        dq[k] = load_io<BF16>(rd, voff, so);
        xq[k] = load_io<BF16>(rx, voff, so);
        if constexpr (FINAL && HAS_Z) zq[k] = load_io<BF16>(rz, voff, so);
        else zq[k] = 0.0f;
    }

    float sumd = 0.0f;
    for (int tb = 0; tb < len; tb += kPrefetch) {
#pragma unroll
        for (int k = 0; k < kPrefetch; ++k) {
            const int t = tb + k;
            if (t >= len) break;
            const float dv = dq[k], xv = xq[k], zv = zq[k];
            {
                const uint32_t so = (uint32_t)min(t + kPrefetch, len - 1) * rstride;
                dq[k] = load_io<BF16>(rd, voff, so);
                xq[k] = load_io<BF16>(rx, voff, so);
                if constexpr (FINAL && HAS_Z) zq[k] = load_io<BF16>(rz, voff, so);
            }
            float Bt[N];
            load_uniform_row<N, BF16>(Bbase, t, Bt);
            const float u = dv * xv;
            if constexpr (FINAL) {
                float Ct[N];
                load_uniform_row<N, BF16>(Cbase, t, Ct);
                float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float ab = exp2_fast(dv * A2[n]);
                    h[n] = __builtin_fmaf(ab, h[n], u * Bt[n]);
                    if (n & 1) y1 = __builtin_fmaf(Ct[n], h[n], y1);
                    else y0 = __builtin_fmaf(Ct[n], h[n], y0);
                }
                float v = y0 + y1;
                if constexpr (HAS_D) v = __builtin_fmaf(Dv, xv, v);
                if constexpr (HAS_Z) v *= silu(zv);
                if (d < D) store_io<BF16>(ry, voff, (uint32_t)t * rstride, v);
            } else {
                sumd += dv;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float ab = exp2_fast(dv * A2[n]);
                    h[n] = __builtin_fmaf(ab, h[n], u * Bt[n]);
                }
            }
        }
    }

    if (d >= D) return;
    if constexpr (FINAL) {
        if (seg == S - 1 && a.h_final != nullptr) {
            float* hp = a.h_final + ((size_t)b * D + d) * N;
#pragma unroll
            for (int n = 0; n < N; ++n) hp[n] = h[n];
        }
    } else {
        float* hout = wsH + (((size_t)b * (S - 1) + seg) * N) * D + d;
#pragma unroll
        for (int n = 0; n < N; ++n) hout[(size_t)n * D] = h[n];
        wsSd[((size_t)b * (S - 1) + seg) * D + d] = sumd;
    }
}

// h_in(s+1) = exp(A sum(Delta_s)) h_in(s) + H_s, s = 0 .. S-2, per (b, n, d).
template <int N>
__global__ void __launch_bounds__(256)
carry_combine(const float* __restrict__ A, const float* __restrict__ h0, float* ws,
              int B, int D, int S) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)B * N * D;
    if (idx >= total) return;
    const int d = (int)(idx % D);
    const int n = (int)((idx / D) % N);
    const int b = (int)(idx / ((size_t)D * N));
    float* wsH = ws;
    const float* wsSd = ws + ws_h_elems(B, S, N, D);
    const float a2 = A[(size_t)d * N + n] * kLog2e;
    float h = h0 ? h0[((size_t)b * D + d) * N + n] : 0.0f;
    constexpr int U = 8;
    for (int s0 = 0; s0 < S - 1; s0 += U) {
        float Hs[U], Sd[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int s = min(s0 + k, S - 2);
            Hs[k] = wsH[(((size_t)b * (S - 1) + s) * N + n) * D + d];
            Sd[k] = wsSd[((size_t)b * (S - 1) + s) * D + d];
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int s = s0 + k;
            if (s >= S - 1) break;
            h = __builtin_fmaf(exp2_fast(a2 * Sd[k]), h, Hs[k]);
            wsH[(((size_t)b * (S - 1) + s) * N + n) * D + d] = h;
        }
    }
}

// L == 0: the final state is the initial state.
__global__ void copy_state(const float* __restrict__ h0, float* __restrict__ out, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

Geom geom(int B, int L, int D, int N) {
    (void)N;
    Geom g;
    const int cw = (D + 63) / 64;                  // channel waves per batch row
    g.threads = 64 * std::min(4, cw);
    const long waves = (long)B * cw;
    const int target = 4096;                       // waves for the final pass
    long S = (target + waves - 1) / waves;
    const int min_len = 32;
    S = std::min<long>(S, std::max<long>(1, (L + min_len - 1) / min_len));
    S = std::max<long>(S, 1);
    int Ls = (int)((L + S - 1) / S);
    if (Ls < 1) Ls = 1;
    g.Ls = Ls;
    g.S = L > 0 ? (L + Ls - 1) / Ls : 0;
    return g;
}

template <int N, bool BF16>
hipError_t launch_n(const ScanArgs& a, hipStream_t st) {
    const Geom g = geom(a.B, a.L, a.D, a.N);
    if (a.L == 0) {
        if (a.h_final) {
            const size_t n = (size_t)a.B * a.D * a.N;
            hipLaunchKernelGGL(copy_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                               a.h0, a.h_final, n);
        }
        return hipGetLastError();
    }
    const dim3 block(g.threads);
    const unsigned gy = (unsigned)((a.D + g.threads - 1) / g.threads);
    if (g.S > 1) {
        hipLaunchKernelGGL((segment_kernel<N, BF16, false, false, false>),
                           dim3(g.S - 1, gy, a.B), block, 0, st, a, g.S, g.Ls);
        const size_t tot = (size_t)a.B * N * a.D;
        hipLaunchKernelGGL(carry_combine<N>, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                           a.A, a.h0, static_cast<float*>(a.ws), a.B, a.D, g.S);
    }
    const dim3 grid(g.S, gy, a.B);
    const bool hz = a.z != nullptr, hd = a.Dskip != nullptr;
    if (hz && hd)
        hipLaunchKernelGGL((segment_kernel<N, BF16, true, true, true>), grid, block, 0, st, a, g.S, g.Ls);
    else if (hz)
        hipLaunchKernelGGL((segment_kernel<N, BF16, true, true, false>), grid, block, 0, st, a, g.S, g.Ls);
    else if (hd)
        hipLaunchKernelGGL((segment_kernel<N, BF16, true, false, true>), grid, block, 0, st, a, g.S, g.Ls);
    else
        hipLaunchKernelGGL((segment_kernel<N, BF16, true, false, false>), grid, block, 0, st, a, g.S, g.Ls);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const ScanArgs& a, hipStream_t st) {
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

bool scan_supported_n(int N) { return N == 4 || N == 8 || N == 16 || N == 32 || N == 64; }

ScanPlan scan_plan(int B, int L, int D, int N) {
    const Geom g = geom(B, L, D, N);
    return ScanPlan{g.S, g.Ls};
}

size_t scan_workspace_bytes(int B, int L, int D, int N) {
    const Geom g = geom(B, L, D, N);
    if (g.S <= 1) return 0;
    return (ws_h_elems(B, g.S, N, D) + (size_t)B * (g.S - 1) * D) * sizeof(float);
}

hipError_t launch_scan_fwd(const ScanArgs& a, hipStream_t st) {
    return a.bf16 ? launch_dtype<true>(a, st) : launch_dtype<false>(a, st);
}

}  // namespace ssm
