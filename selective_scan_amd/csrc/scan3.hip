// Mamba-3 selective scan on gfx950: complex diagonal transitions A = Are + i theta
// and the exponential-trapezoidal rule ("Efficient Sequence Modeling: From S4 to
// Mamba-3", section 03 System, mamba3_minimal.py; section 04 "Complex transitions
// for state tracking"). Per (batch, channel), complex state h[n]:
//   alpha_t = exp(Delta_t (Are + i theta))
//   h_t     = alpha_t h_{t-1} + (1 - lam_t) Delta_t alpha_t B_{t-1} x_{t-1} + lam_t Delta_t B_t x_t
//   y_t     = (sum_n C_t[n] Re h_t[n] + D x_t) silu(z_t)
// The two input terms are the trapezoidal rule, weighted by lam_t, on the exact
// one-step integral of e^{A (Delta - s)} B x; lam = 1, theta = 0 is the plain
// exponential-Euler scan. B_{-1} x_{-1} is the token before the sequence (x_prev,
// B_prev), zero when absent.
//
// Work mapping: the plain scan's (one lane per (batch, channel), the N complex
// states in VGPRs as real and imaginary parts, B and C rows wave-uniform in SGPRs
// through scalar loads), and its L-parallel structure in three launches:
//   1. seg_agg3: every segment from a zero state; in LDS each segment's exclusive
//      in-group prefix (the state its group's earlier segments leave) and the
//      group's aggregate. A segment's input includes its first step's trapezoid
//      term, read from the token before the segment.
//   2. carry3: per (batch, state, channel) the state entering each group.
//   3. seg_final3: the recurrence again from the carried-in state, writing y.
// One group of segments (seg_fused3) runs all three in one launch.
// Segments compose as affine maps with complex coefficients: (P1, H1) then
// (P2, H2) = (P2 P1, P2 H1 + H2), P = exp(A sum Delta) = 2^{Are' S} (cos, sin)(theta S).
// alpha takes v_exp_f32, v_sin_f32 and v_cos_f32 (the last two in revolutions).
#include "common.h"
#include "scan3.h"

#include <algorithm>

namespace ssm {
namespace {

constexpr int kW3 = 4;            // segments (waves) per workgroup
// waves the passes aim for: B8 L32768 D512, 2.27 ms per call at 4096, 2.17 at 8192, 2.11
// at 16384 and 2.12-2.13 at 24576 and 32768 (longer carries); shorter sequences are
// bound by the shortest segment instead
constexpr int kTarget3 = 16384;
constexpr int kMinSeg3 = 32;      // shortest segment
constexpr float kInv2Pi = 0.15915494309189535f;

struct Geom3 {
    int Ls, S, G;
};

Geom3 geom3(int B, int L, int D) {
    Geom3 g{1, 0, 0};
    if (L <= 0) return g;
    const long chains = (long)B * ((D + 63) / 64);
    const long st = std::max<long>(1, (kTarget3 + chains - 1) / chains);
    long Ls = std::max<long>(kMinSeg3, (L + st - 1) / st);
    Ls = std::min<long>(Ls, L);
    g.Ls = (int)Ls;
    g.S = (int)((L + Ls - 1) / Ls);
    g.G = (g.S + kW3 - 1) / kW3;
    return g;
}

// workspace (floats), channel index fastest:
//   E  [B][S][2][N][D]  exclusive in-group prefix state of each segment (re, im)
//   CS [B][S][D]        in-group prefix of sum(Delta) before each segment
//   GH [B][G-1][2][N][D] aggregate of each group (from zero); carry3 overwrites slot g
//                        with the state entering group g + 1
//   GS [B][G-1][D]      sum(Delta) over each group
struct Ws3 {
    size_t E, CS, GH, GS, total;
};

__host__ __device__ inline Ws3 ws3(int B, int D, int N, int S, int G) {
    Ws3 w;
    const size_t g1 = G > 1 ? (size_t)(G - 1) : 0;
    w.E = 0;
    w.CS = w.E + (size_t)B * S * 2 * N * D;
    w.GH = w.CS + (size_t)B * S * D;
    w.GS = w.GH + (size_t)B * g1 * 2 * N * D;
    w.total = w.GS + (size_t)B * g1 * D;
    return w;
}

template <bool BF16>
__device__ __forceinline__ float ld_io(const void* p, size_t i) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}

// One step's complex decay exp(dv (Are + i theta)) with A2 = Are log2 e and th =
// theta / (2 pi) (revolutions; one step turns far less than a revolution).
__device__ __forceinline__ void cstep(float dv, float A2, float th, float& pr, float& pi) {
    const float m = exp2_fast(dv * A2);
    const float ph = dv * th;
    pr = m * __builtin_amdgcn_cosf(ph);
    pi = m * __builtin_amdgcn_sinf(ph);
}

// The same over a sum of many steps s, with the phase first reduced to
// [-1/2, 1/2] revolution, where v_sin / v_cos are most accurate.
__device__ __forceinline__ void cdecay(float s, float A2, float th, float& pr, float& pi) {
    const float m = exp2_fast(s * A2);
    float ph = s * th;
    ph -= __builtin_rintf(ph);
    pr = m * __builtin_amdgcn_cosf(ph);
    pi = m * __builtin_amdgcn_sinf(ph);
}

// One wave's walk over steps [t0, t0 + len) of its 64 channels. FINAL: also the
// outputs. The state (hr, hi) is updated in place; sumd accumulates Delta.
template <int N, bool BF16, bool FINAL>
__device__ __forceinline__ void walk3(const Scan3Args& a, int b, int d, int dc, int t0, int len, const float (&A2)[N],
                                      const float (&th)[N], float (&hr)[N], float (&hi)[N], float Dv,
                                      float& sumd) {
    const int D = a.D, NT = a.N;
    const int rw = BF16 ? NT / 2 : NT;
    // the token before the segment: the previous step's x and B row, or x_prev /
    // B_prev at the sequence start (zero when absent)
    Row<N, BF16> Bp, Bt, Ct;
    float xp = 0.0f;
    bool have_prev = true;
    if (t0 > 0) {
        const size_t row = (size_t)b * a.L + t0 - 1;
        xp = ld_io<BF16>(a.x, row * D + dc);
        Bp.load(a.Bm, (long)row, rw);
    } else if (a.x_prev != nullptr) {
        xp = ld_io<BF16>(a.x_prev, (size_t)b * D + dc);
        Bp.load(a.B_prev, (long)b, rw);
    } else {
        have_prev = false;
    }
    if (!have_prev) {
#pragma unroll
        for (int k = 0; k < Row<N, BF16>::K; ++k) Bp.v[k] = 0u;
    }
    // this step's x, Delta, lam (and z) were loaded one step earlier
    auto at = [&](int t) { return ((size_t)b * a.L + t0 + t) * D + dc; };
    float dn = ld_io<BF16>(a.delta, at(0)), xn = ld_io<BF16>(a.x, at(0)), ln = ld_io<BF16>(a.lam, at(0));
    float zn = (FINAL && a.z != nullptr) ? ld_io<BF16>(a.z, at(0)) : 0.0f;
    for (int t = 0; t < len; ++t) {
        const size_t row = (size_t)b * a.L + t0 + t;
        const size_t i = row * D + dc;
        const float dv = dn, xv = xn, lv = ln, zv = zn;
        {
            const size_t j = at(min(t + 1, len - 1));
            dn = ld_io<BF16>(a.delta, j);
            xn = ld_io<BF16>(a.x, j);
            ln = ld_io<BF16>(a.lam, j);
            if (FINAL && a.z != nullptr) zn = ld_io<BF16>(a.z, j);
        }
        Bt.load(a.Bm, (long)row, rw);
        if constexpr (FINAL) Ct.load(a.Cm, (long)row, rw);
        const float q = (1.0f - lv) * dv * xp;  // weight of B_{t-1}[n] (times alpha)
        const float r = lv * dv * xv;           // weight of B_t[n]
        float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            float ar, ai;
            cstep(dv, A2[n], th[n], ar, ai);
            const float g = __builtin_fmaf(q, Bp.at(n), hr[n]);  // h + q B_{t-1}: both multiplied by alpha
            const float nr = __builtin_fmaf(ar, g, __builtin_fmaf(-ai, hi[n], r * Bt.at(n)));
            const float ni = __builtin_fmaf(ai, g, ar * hi[n]);
            hr[n] = nr;
            hi[n] = ni;
            if constexpr (FINAL) {
                if (n & 1) y1 = __builtin_fmaf(Ct.at(n), nr, y1);
                else y0 = __builtin_fmaf(Ct.at(n), nr, y0);
            }
        }
        if constexpr (FINAL) {
            float v = __builtin_fmaf(Dv, xv, y0 + y1);
            if (a.z != nullptr) v *= silu(zv);
            if (d < D) {
                if constexpr (BF16) static_cast<uint16_t*>(a.y)[i] = f32_to_bf16(v);
                else static_cast<float*>(a.y)[i] = v;
            }
        } else {
            sumd += dv;
        }
        Bp = Bt;
        xp = xv;
    }
}

template <int N, bool BF16>
__global__ void __launch_bounds__(64 * kW3) seg_agg3(Scan3Args a, Geom3 g) {
    // Each wave's end state and sum of Delta go through LDS; its decay
    // exp(sum Delta (Are + i theta)) is recomputed by the waves that need it (the same
    // lane holds the same channel's Are and theta), which halves the LDS a workgroup
    // takes (33 KB) and lets three workgroups share a CU instead of two.
    __shared__ float sHr[kW3][N][64], sHi[kW3][N][64], sS[kW3][64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = blockIdx.x, b = blockIdx.z;
    const int D = a.D;
    const int d = blockIdx.y * 64 + lane, dc = d < D ? d : D - 1;
    const int s = grp * kW3 + wave;
    const int t0 = s * g.Ls;
    const int len = s < g.S ? min(g.Ls, a.L - t0) : 0;
    float A2[N], th[N], hr[N], hi[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.Are[(size_t)dc * N + n] * kLog2e;
        th[n] = a.theta[(size_t)dc * N + n] * kInv2Pi;
        hr[n] = 0.0f;
        hi[n] = 0.0f;
    }
    float sumd = 0.0f;
    if (len > 0) walk3<N, BF16, false>(a, b, d, dc, t0, len, A2, th, hr, hi, 0.0f, sumd);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        sHr[wave][n][lane] = hr[n];
        sHi[wave][n][lane] = hi[n];
    }
    sS[wave][lane] = sumd;
    __syncthreads();
    // exclusive in-group prefix: E_{j+1} = P_j E_j + H_j
    float er[N], ei[N];
#pragma unroll
    for (int n = 0; n < N; ++n) er[n] = ei[n] = 0.0f;
    float cs = 0.0f;
    for (int j = 0; j < wave; ++j) {
        const float sj = sS[j][lane];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            float pr, pi;
            cdecay(sj, A2[n], th[n], pr, pi);
            const float nr = pr * er[n] - pi * ei[n] + sHr[j][n][lane];
            const float ni = pr * ei[n] + pi * er[n] + sHi[j][n][lane];
            er[n] = nr;
            ei[n] = ni;
        }
        cs += sj;
    }
    if (d >= D || s >= g.S) return;
    const Ws3 wl = ws3(a.B, D, N, g.S, g.G);
    float* ws = static_cast<float*>(a.ws);
    if (wave > 0) {
        float* Ep = ws + wl.E + ((size_t)b * g.S + s) * 2 * N * D + d;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            Ep[(size_t)n * D] = er[n];
            Ep[(size_t)(N + n) * D] = ei[n];
        }
        ws[wl.CS + ((size_t)b * g.S + s) * D + d] = cs;
    }
    const bool last_in_group = (wave == kW3 - 1) || (s == g.S - 1);
    if (last_in_group && grp < g.G - 1) {
        float* GH = ws + wl.GH + ((size_t)b * (g.G - 1) + grp) * 2 * N * D + d;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            float pr, pi;
            cdecay(sumd, A2[n], th[n], pr, pi);
            GH[(size_t)n * D] = pr * er[n] - pi * ei[n] + hr[n];
            GH[(size_t)(N + n) * D] = pr * ei[n] + pi * er[n] + hi[n];
        }
        ws[wl.GS + ((size_t)b * (g.G - 1) + grp) * D + d] = cs + sumd;
    }
}

// state entering each group: carry(0) = h0, carry(g+1) = P_g carry(g) + H_g, written
// over H_g. One thread per (batch, state, channel); the groups in order.
template <int N>
__global__ void __launch_bounds__(256) carry3(Scan3Args a, Geom3 g) {
    const int d = blockIdx.x * 256 + threadIdx.x, n = blockIdx.y, b = blockIdx.z;
    const int D = a.D;
    if (d >= D) return;
    const Ws3 wl = ws3(a.B, D, N, g.S, g.G);
    float* ws = static_cast<float*>(a.ws);
    const float A2 = a.Are[(size_t)d * N + n] * kLog2e, th = a.theta[(size_t)d * N + n] * kInv2Pi;
    float hr = 0.0f, hi = 0.0f;
    if (a.h0 != nullptr) {
        hr = a.h0[(((size_t)b * D + d) * N + n) * 2];
        hi = a.h0[(((size_t)b * D + d) * N + n) * 2 + 1];
    }
    // U groups' aggregates loaded before any is chained (one memory round trip per U
    // groups: a load after the previous group's store would wait for it)
    constexpr int U = 8;
    const int steps = g.G - 1;
    for (int k0 = 0; k0 < steps; k0 += U) {
        float gs[U], vr[U], vi[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = min(k0 + u, steps - 1);
            const float* GH = ws + wl.GH + ((size_t)b * (g.G - 1) + k) * 2 * N * D + d;
            gs[u] = ws[wl.GS + ((size_t)b * (g.G - 1) + k) * D + d];
            vr[u] = GH[(size_t)n * D];
            vi[u] = GH[(size_t)(N + n) * D];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k0 + u >= steps) break;
            float* GH = ws + wl.GH + ((size_t)b * (g.G - 1) + k0 + u) * 2 * N * D + d;
            float pr, pi;
            cdecay(gs[u], A2, th, pr, pi);
            const float nr = pr * hr - pi * hi + vr[u];
            const float ni = pr * hi + pi * hr + vi[u];
            hr = nr;
            hi = ni;
            GH[(size_t)n * D] = hr;
            GH[(size_t)(N + n) * D] = hi;
        }
    }
}

template <int N, bool BF16>
__global__ void __launch_bounds__(64 * kW3) seg_final3(Scan3Args a, Geom3 g) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = blockIdx.x, b = blockIdx.z;
    const int D = a.D;
    const int d = blockIdx.y * 64 + lane, dc = d < D ? d : D - 1;
    const int s = grp * kW3 + wave;
    if (s >= g.S) return;
    const int t0 = s * g.Ls, len = min(g.Ls, a.L - t0);
    const Ws3 wl = ws3(a.B, D, N, g.S, g.G);
    const float* ws = static_cast<const float*>(a.ws);
    float A2[N], th[N], hr[N], hi[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.Are[(size_t)dc * N + n] * kLog2e;
        th[n] = a.theta[(size_t)dc * N + n] * kInv2Pi;
    }
    // state entering the group
    float gr[N], gi[N];
    if (grp > 0) {
        const float* GH = ws + wl.GH + ((size_t)b * (g.G - 1) + grp - 1) * 2 * N * D + dc;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            gr[n] = GH[(size_t)n * D];
            gi[n] = GH[(size_t)(N + n) * D];
        }
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            gr[n] = a.h0 ? a.h0[(((size_t)b * D + dc) * N + n) * 2] : 0.0f;
            gi[n] = a.h0 ? a.h0[(((size_t)b * D + dc) * N + n) * 2 + 1] : 0.0f;
        }
    }
    // h_in = exp(A cs) h_group + E_s
    float cs = 0.0f;
    if (wave > 0) cs = ws[wl.CS + ((size_t)b * g.S + s) * D + dc];
    const float* Ep = ws + wl.E + ((size_t)b * g.S + s) * 2 * N * D + dc;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        float pr, pi;
        cdecay(cs, A2[n], th[n], pr, pi);
        const float er = wave > 0 ? Ep[(size_t)n * D] : 0.0f, ei = wave > 0 ? Ep[(size_t)(N + n) * D] : 0.0f;
        hr[n] = pr * gr[n] - pi * gi[n] + er;
        hi[n] = pr * gi[n] + pi * gr[n] + ei;
    }
    const float Dv = a.Dskip ? a.Dskip[dc] : 0.0f;
    float unused = 0.0f;
    walk3<N, BF16, true>(a, b, d, dc, t0, len, A2, th, hr, hi, Dv, unused);
    if (d < D && s == g.S - 1 && a.h_final != nullptr) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            a.h_final[(((size_t)b * D + d) * N + n) * 2] = hr[n];
            a.h_final[(((size_t)b * D + d) * N + n) * 2 + 1] = hi[n];
        }
    }
}

// A short sequence (2 .. kW3 segments, one group): one launch. Each wave runs its
// segment from a zero state, the waves meet in LDS for the exclusive prefix of the
// earlier segments (end states and sums of Delta; decays recomputed), and each wave
// runs its segment again from its entering state (h0 folded in). No workspace.
template <int N, bool BF16>
__global__ void __launch_bounds__(64 * kW3) seg_fused3(Scan3Args a, Geom3 g) {
    __shared__ float sHr[kW3][N][64], sHi[kW3][N][64], sS[kW3][64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int b = blockIdx.z, D = a.D;
    const int d = blockIdx.y * 64 + lane, dc = d < D ? d : D - 1;
    const int s = wave;
    const int t0 = s * g.Ls;
    const int len = s < g.S ? min(g.Ls, a.L - t0) : 0;
    float A2[N], th[N], hr[N], hi[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.Are[(size_t)dc * N + n] * kLog2e;
        th[n] = a.theta[(size_t)dc * N + n] * kInv2Pi;
        hr[n] = 0.0f;
        hi[n] = 0.0f;
    }
    float sumd = 0.0f;
    if (len > 0) walk3<N, BF16, false>(a, b, d, dc, t0, len, A2, th, hr, hi, 0.0f, sumd);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        sHr[wave][n][lane] = hr[n];
        sHi[wave][n][lane] = hi[n];
    }
    sS[wave][lane] = sumd;
    __syncthreads();
    if (len == 0) return;
    float er[N], ei[N];
#pragma unroll
    for (int n = 0; n < N; ++n) er[n] = ei[n] = 0.0f;
    float cs = 0.0f;
    for (int j = 0; j < wave; ++j) {
        const float sj = sS[j][lane];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            float pr, pi;
            cdecay(sj, A2[n], th[n], pr, pi);
            const float nr = pr * er[n] - pi * ei[n] + sHr[j][n][lane];
            const float ni = pr * ei[n] + pi * er[n] + sHi[j][n][lane];
            er[n] = nr;
            ei[n] = ni;
        }
        cs += sj;
    }
    // h_in = exp(A cs) h0 + E
#pragma unroll
    for (int n = 0; n < N; ++n) {
        if (a.h0 != nullptr) {
            const float gr = a.h0[(((size_t)b * D + dc) * N + n) * 2], gi = a.h0[(((size_t)b * D + dc) * N + n) * 2 + 1];
            float pr, pi;
            cdecay(cs, A2[n], th[n], pr, pi);
            hr[n] = pr * gr - pi * gi + er[n];
            hi[n] = pr * gi + pi * gr + ei[n];
        } else {
            hr[n] = er[n];
            hi[n] = ei[n];
        }
    }
    const float Dv = a.Dskip ? a.Dskip[dc] : 0.0f;
    float unused = 0.0f;
    walk3<N, BF16, true>(a, b, d, dc, t0, len, A2, th, hr, hi, Dv, unused);
    if (d < D && s == g.S - 1 && a.h_final != nullptr) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            a.h_final[(((size_t)b * D + d) * N + n) * 2] = hr[n];
            a.h_final[(((size_t)b * D + d) * N + n) * 2 + 1] = hi[n];
        }
    }
}

// L == 0: the final state is the initial state.
__global__ void copy_state3(const float* __restrict__ h0, float* __restrict__ out, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

template <int N, bool BF16>
hipError_t launch3(const Scan3Args& a, hipStream_t st) {
    const Geom3 g = geom3(a.B, a.L, a.D);
    if (a.L == 0) {
        if (a.h_final) {
            const size_t n = (size_t)a.B * a.D * a.N * 2;
            launch(copy_state3, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.h0, a.h_final, n);
        }
        return hipGetLastError();
    }
    if (g.S > 1 && g.G == 1) {
        launch((seg_fused3<N, BF16>), dim3(1, (unsigned)((a.D + 63) / 64), (unsigned)a.B), dim3(64 * g.S), 0, st,
               a, g);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)g.G, (unsigned)((a.D + 63) / 64), (unsigned)a.B);
    if (g.S > 1) launch((seg_agg3<N, BF16>), grid, dim3(64 * kW3), 0, st, a, g);
    if (g.G > 1)
        launch((carry3<N>), dim3((unsigned)((a.D + 255) / 256), (unsigned)N, (unsigned)a.B), dim3(256), 0, st, a, g);
    launch((seg_final3<N, BF16>), grid, dim3(64 * kW3), 0, st, a, g);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch3_n(const Scan3Args& a, hipStream_t st) {
    switch (a.N) {
        case 4: return launch3<4, BF16>(a, st);
        case 8: return launch3<8, BF16>(a, st);
        case 16: return launch3<16, BF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool scan3_supported_n(int N) { return N == 4 || N == 8 || N == 16; }

int scan3_segment_len(int B, int L, int D) { return geom3(B, L, D).Ls; }

size_t scan3_workspace_bytes(int B, int L, int D, int N) {
    const Geom3 g = geom3(B, L, D);
    if (g.S <= 1 || g.G == 1) return 0;  // one segment, or one group run in one launch
    return ws3(B, D, N, g.S, g.G).total * sizeof(float);
}

hipError_t launch_scan3_fwd(const Scan3Args& a, hipStream_t st) {
    return a.bf16 ? launch3_n<true>(a, st) : launch3_n<false>(a, st);
}

}  // namespace ssm
