// Mamba-1 selective scan kernels on gfx950, shared by the plain forward entry point
// (scan_fwd.hip) and its discretisation variants (scan_var.hip).
// The scan: h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t,
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
// L-parallelism. B*D channels alone cannot fill 256 CUs, so each chain of 64
// channels is cut into S segments of Ls steps; W consecutive segments form a
// group, handled by one workgroup of W waves (one wave per segment). Three launches:
//   1. segment_aggregate: every wave runs its segment from a zero state (end
//      state H_s, sum of Delta; its decay P_s = exp(A sum Delta) is recomputed
//      where needed); the group's waves then form, in LDS, each segment's
//      exclusive in-group prefix E_s (and the in-group prefix of sum Delta), and
//      the last wave the group's own aggregate (GP_g, GH_g).
//   2. group_carry: per (batch, channel, state index) the state entering each
//      group, from the groups' aggregates (a two-level walk over the groups).
//   3. segment_final: each wave forms its segment's carried-in state
//      h_in = exp(A * prefix sum Delta) h_group + E_s and runs the recurrence
//      again from it, writing y (and h_final at the end of the sequence).
// (P1, H1) then (P2, H2) compose to (P2 P1, P2 H1 + H2): the recurrence is an
// affine map of the state, so segments compose like affine maps. A short chain
// (segment_fused) runs all three steps in one launch, one workgroup per chain.
//
// N >= 64 (64, 128, 256): a lane's 64 states and 64 entries of A would fill its
// registers, so the state index is cut into chunks of 16 that run as independent
// chains (aggregate, carry and recurrence are independent across state indices);
// the final pass (segment_final_sink: one workgroup holds up to 8 chunk waves of a
// segment and 64 channels) adds the chunks' partial C . h in LDS; with every chunk
// in the workgroup (N <= 128) it finishes y there, else it writes one fp32 sum per
// (t, channel) and chunk group and a fourth launch (combine_partials) adds the
// groups' sums, the skip and the gate.
#pragma once
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace ssm {
namespace {

// Geometry defaults; each can be overridden at build time (-DSSM_SCAN_...).
#ifndef SSM_SCAN_PREFETCH
#define SSM_SCAN_PREFETCH 4
#endif
#ifndef SSM_SCAN_PREFETCH_FINAL
#define SSM_SCAN_PREFETCH_FINAL 2
#endif
#ifndef SSM_SCAN_TARGET_WAVES
#define SSM_SCAN_TARGET_WAVES 16384
#endif
#ifndef SSM_SCAN_MIN_SEGMENT
#define SSM_SCAN_MIN_SEGMENT 32
#endif
#ifndef SSM_SCAN_MAX_GROUP
#define SSM_SCAN_MAX_GROUP 4
#endif
// Steps of x/Delta/z in flight per lane: kPrefetch in the aggregate pass and the
// chunked (N >= 64) final pass, kPrefetchFinal in the plain final pass. Fewer
// registers in the ring buy waves, and with 16384 target waves (three or more
// waves per SIMD over the launch) the waves hide the load latency better than a
// deep ring: B8 L32768 D512 N16 went from 0.72 ms per call (5120 waves, ring of 8)
// to 0.64 ms (aggregate 287 -> 269 us, final 427 -> 356 us); at B1 L4096 D1536
// N16 0.051 -> 0.049 ms; N = 64 unchanged.
constexpr int kPrefetch = SSM_SCAN_PREFETCH;
constexpr int kPrefetchFinal = SSM_SCAN_PREFETCH_FINAL;
constexpr int kTargetWaves = SSM_SCAN_TARGET_WAVES;  // waves the final pass aims for
constexpr int kMinSegment = SSM_SCAN_MIN_SEGMENT;    // shortest segment (steps)

struct Geom {
    int Ls;  // steps per segment
    int S;   // segments per chain
    int W;   // segments (waves) per workgroup
    int G;   // groups per chain
};

#ifndef SSM_SCAN_CHUNK_N
#define SSM_SCAN_CHUNK_N 16
#endif
#ifndef SSM_SCAN_CHUNK_WAVES
#define SSM_SCAN_CHUNK_WAVES 16384
#endif
// N >= 64 runs as N / kChunkN independent chains of kChunkN states per lane (a sweep
// of 16/32/64 states per lane and 2048-16384 target waves on the N = 64, 128, 256
// sweep shapes put 16 and 16384 first: the short chains keep ~80 VGPRs and several
// waves per SIMD, which outweighs the extra partial sums they write).
constexpr int kChunkN = SSM_SCAN_CHUNK_N;
constexpr int kChunkWaves = SSM_SCAN_CHUNK_WAVES;  // waves the chunked passes aim for
inline int n_chunks(int N) { return N >= 64 ? N / kChunkN : 1; }
inline int lane_states(int N) { return n_chunks(N) > 1 ? kChunkN : N; }
inline int max_group(int N) { return std::max(1, std::min(SSM_SCAN_MAX_GROUP, 128 / lane_states(N))); }

Geom geom(int B, int L, int D, int N) {
    Geom g{1, 0, 1, 0};
    if (L <= 0) return g;
    const long chains = (long)B * ((D + 63) / 64) * n_chunks(N);
    const long s_target = n_chunks(N) > 1 ? std::max<long>(1, kChunkWaves / chains)
                                          : (kTargetWaves + chains - 1) / chains;
    long Ls = std::max<long>(kMinSegment, (L + s_target - 1) / s_target);
    Ls = std::min<long>(Ls, L);
    g.Ls = (int)Ls;
    g.S = (int)((L + Ls - 1) / Ls);
    g.W = std::min(max_group(N), g.S);
    g.G = (g.S + g.W - 1) / g.W;
    return g;
}

// workspace layout (floats), all with the channel index fastest:
//   E  [B][S][N][D]   exclusive in-group prefix state of each segment
//   CS [B][S][D]      in-group prefix of sum(Delta) before each segment
//   GH [B][G-1][N][D] aggregate end state of each group (from zero); group_carry
//                     overwrites slot g with the state entering group g+1
//   GP [B][G-1][N][D] aggregate decay of each group
//   YP [P][B][L][D]   fp32 C . h summed over each group of up to 8 state chunks
//                     (P = sink_planes(N) groups; N >= 64 only)
struct WsLayout {
    size_t E, CS, GH, GP, YP, total;
};

__host__ __device__ inline WsLayout ws_layout(int B, int D, int N, int S, int G) {
    WsLayout w;
    const size_t g1 = G > 1 ? (size_t)(G - 1) : 0;
    w.E = 0;
    w.CS = w.E + (size_t)B * S * N * D;
    w.GH = w.CS + (size_t)B * S * D;
    w.GP = w.GH + (size_t)B * g1 * N * D;
    w.YP = w.GP + (size_t)B * g1 * N * D;
    w.total = w.YP;
    return w;
}

// Discretisation variants (template parameter V of the segment kernels):
//   V = 0  exponential-Euler, Delta as given (the plain path);
//   V = 1  exponential-Euler, Delta = [softplus](delta + bias);
//   V = 2  exact zero-order hold, Delta = [softplus](delta + bias).
// Zero-order hold ("Efficient Sequence Modeling: From S4 to Mamba-3", section 04
// and Q01): Bbar x = Delta B x (e^z - 1)/z = (e^z - 1)/A B x with z = Delta A. A step
// whose |z| >= kZohSmall for every lane and state takes h' = e^z (h + w) - w with
// w = x B / A (no rounding worse than 2 ulp / kZohSmall); otherwise the wave takes
// the blended form, (e^z - 1)/A where |z| >= kZohSmall and Delta (1 + z/2 + z^2/6 +
// z^3/24) below it (truncation < 1e-8 relative), which also covers A = 0.
constexpr float kZohSmall = 0.03125f;
constexpr float kZohSmall2 = kZohSmall * kLog2e;  // the same bound on |Delta A log2 e|
constexpr float kLn2f = 0.69314718055994531f;
// (ln 2)^k / (k+1)!, k = 1, 2, 3: the series 1 + z/2 + z^2/6 + z^3/24 in z2 = z log2 e
constexpr double kLn2d = 0.69314718055994531;
constexpr float kZohT1 = (float)(kLn2d / 2.0);
constexpr float kZohT2 = (float)(kLn2d * kLn2d / 6.0);
constexpr float kZohT3 = (float)(kLn2d * kLn2d * kLn2d / 24.0);

template <int N, int V>
struct VarLane {};  // V = 0: nothing per lane
template <int N>
struct VarLane<N, 1> {
    float bias;
    bool softplus;
};
template <int N>
struct VarLane<N, 2> {
    float bias;
    bool softplus;
    float rA[N];  // 1 / A (inf for A = 0: only read where |z| >= kZohSmall)
    float amin2;  // min over the lane's states of |A log2 e|
};

template <int N, int V>
__device__ __forceinline__ void var_lane_init(VarLane<N, V>& vl, const ScanArgs& a, int dc, int n0) {
    if constexpr (V >= 1) {
        vl.bias = a.delta_bias != nullptr ? a.delta_bias[dc] : 0.0f;
        vl.softplus = a.delta_softplus != 0;
    }
    if constexpr (V == 2) {
        vl.amin2 = __builtin_inff();
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float A = a.A[(size_t)dc * a.N + n0 + n];
            vl.rA[n] = 1.0f / A;
            vl.amin2 = fminf(vl.amin2, fabsf(A) * kLog2e);
        }
    }
}

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|), with log1p by its series
// below 1/64 (error < 2e-8 relative) and by v_log_f32 above.
__device__ __forceinline__ float softplus_f(float v) {
    const float e = exp2_fast(-fabsf(v) * kLog2e);
    const float series = e * __builtin_fmaf(e, __builtin_fmaf(e, 1.0f / 3.0f, -0.5f), 1.0f);
    const float lg = __builtin_amdgcn_logf(1.0f + e) * kLn2f;
    return fmaxf(v, 0.0f) + (e < 0.015625f ? series : lg);
}

template <int N, int V>
__device__ __forceinline__ float var_delta(float dv, const VarLane<N, V>& vl) {
    if constexpr (V == 0) {
        return dv;
    } else {
        const float v = dv + vl.bias;
        return vl.softplus ? softplus_f(v) : v;
    }
}

// One wave's segment of the recurrence. Construction issues the first loads
// (kP steps of x, Delta[, z] and the first B[, C] rows), so a caller can
// start them before other prologue work; run() then walks the segment.
template <int N, bool BF16, bool HAS_Z, bool HAS_D, bool FINAL, int V = 0, bool SINK = false>
struct Segment {
    static_assert(!SINK || FINAL, "the LDS sink holds the final pass's partial sums");
    static constexpr uint32_t es = BF16 ? 2 : 4;
    // ring depth; the LDS sink's slot layout is sized with kPrefetch
    static constexpr int kP = FINAL && !SINK ? kPrefetchFinal : kPrefetch;
    static constexpr bool kZ = FINAL && HAS_Z;
    __amdgpu_buffer_rsrc_t rx, rd, rz, ry;
    uint32_t voff, yoff, rstride, ystride;
    const void* Bbase;
    const void* Cbase;
    int rw;  // row stride of B and C in 32-bit words
    int len;
    float* lsink = nullptr;  // SINK: ring slot k's partial sums go to lsink[64 k + lane]
    uint32_t dq[kP], xq[kP], zq[kP];
    Row<N, BF16> Bn, Cn;

    // store: this lane's channel exists (d < D); other lanes aim their y stores
    // past the end of the y view, where the buffer unit drops them (no branch).
    // The lane's states are n0 .. n0 + N - 1 of a.N. SINK: the fp32 C . h of these
    // states only goes to LDS (lsink) instead of y.
    __device__ __forceinline__ Segment(const ScanArgs& a, int b, int dc, int t0, int len_, int n0,
                                       bool store = true)
        : len(len_) {
        const size_t row0 = (size_t)b * a.L + t0;
        const uint32_t bytes = (uint32_t)len * (uint32_t)a.D * es;
        const char* xb = static_cast<const char*>(a.x) + row0 * a.D * es;
        rx = make_rsrc(xb, bytes);
        rd = make_rsrc(static_cast<const char*>(a.delta) + row0 * a.D * es, bytes);
        rz = make_rsrc(kZ ? static_cast<const char*>(a.z) + row0 * a.D * es : xb, bytes);
        ry = make_rsrc(FINAL ? static_cast<const char*>(a.y) + row0 * a.D * es : xb, bytes);
        yoff = store ? (uint32_t)dc * es : 0x80000000u;
        ystride = (uint32_t)a.D * es;
        voff = (uint32_t)dc * es;
        rstride = (uint32_t)a.D * es;
        Bbase = static_cast<const char*>(a.Bm) + (row0 * a.N + n0) * es;
        Cbase = static_cast<const char*>(a.Cm) + (row0 * a.N + n0) * es;
        rw = BF16 ? a.N / 2 : a.N;
#pragma unroll
        for (int k = 0; k < kP; ++k) {
            const uint32_t so = (uint32_t)min(k, len - 1) * rstride;
            dq[k] = load_raw<BF16>(rd, voff, so);
            xq[k] = load_raw<BF16>(rx, voff, so);
            zq[k] = kZ ? load_raw<BF16>(rz, voff, so) : 0u;
        }
        Bn.load(Bbase, 0, rw);
        if constexpr (FINAL) Cn.load(Cbase, 0, rw);
    }

    // the input term of state n for one step: h' = a h + Bbar x
    template <int MODE>
    __device__ __forceinline__ float update(float hv, float ab, float dv, float xv, float u, float b, float a2,
                                            const VarLane<N, V>& vl, int n) const {
        if constexpr (V < 2) {
            return __builtin_fmaf(ab, hv, u * b);
        } else if constexpr (MODE == 0) {  // every |z| >= kZohSmall in the wave
            const float w = xv * vl.rA[n] * b;
            return __builtin_fmaf(ab, hv + w, -w);
        } else {
            // coef = Delta (e^z - 1)/z: the series in z2 = z log2 e (coefficients
            // (ln 2)^k / (k+1)! folded in) below the switch, (e^z - 1)/A as
            // ab/A - 1/A in one fma above it
            const float z2 = dv * a2;
            const float taylor = dv * __builtin_fmaf(z2, __builtin_fmaf(z2, __builtin_fmaf(z2, kZohT3, kZohT2), kZohT1),
                                                     1.0f);
            const float coef = fabsf(z2) < kZohSmall2 ? taylor : __builtin_fmaf(ab, vl.rA[n], -vl.rA[n]);
            return __builtin_fmaf(ab, hv, coef * (xv * b));
        }
    }

    template <int MODE>
    __device__ __forceinline__ void states(const float (&A2)[N], float (&h)[N], float dv, float xv,
                                           const Row<N, BF16>& Bt, const Row<N, BF16>& Ct, const VarLane<N, V>& vl,
                                           float& y0, float& y1) const {
        const float u = dv * xv;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float ab = exp2_fast(dv * A2[n]);
            h[n] = update<MODE>(h[n], ab, dv, xv, u, Bt.at(n), A2[n], vl, n);
            if constexpr (FINAL) {
                if (n & 1) y1 = __builtin_fmaf(Ct.at(n), h[n], y1);
                else y0 = __builtin_fmaf(Ct.at(n), h[n], y0);
            }
        }
    }

    // one time step t from ring slot k; RELOAD: refill the slot with step t + kP
    template <bool RELOAD>
    __device__ __forceinline__ void step(int t, int k, const float (&A2)[N], float (&h)[N], float Dv,
                                         float& sumd, const VarLane<N, V>& vl) {
        const float dv = var_delta<N, V>(widen<BF16>(dq[k]), vl), xv = widen<BF16>(xq[k]);
        const float zv = kZ ? widen<BF16>(zq[k]) : 0.0f;
        if constexpr (RELOAD) {
            const uint32_t so = (uint32_t)min(t + kP, len - 1) * rstride;
            dq[k] = load_raw<BF16>(rd, voff, so);
            xq[k] = load_raw<BF16>(rx, voff, so);
            if constexpr (kZ) zq[k] = load_raw<BF16>(rz, voff, so);
        }
        const Row<N, BF16> Bt = Bn;
        Row<N, BF16> Ct;
        if constexpr (FINAL) Ct = Cn;
        const int tn = min(t + 1, len - 1);
        Bn.load(Bbase, tn, rw);
        if constexpr (FINAL) Cn.load(Cbase, tn, rw);
        // The aggregate pass pins the next step's B row load here, a whole step ahead
        // of its use: left alone, the scheduler sinks each scalar load to just before
        // its first use and every step waits out its latency (B8 L32768 D512 N16:
        // 340 -> 287 us per launch, bitwise the same). The final pass holds the C rows
        // as well; there the barrier leaves too few SGPRs and was slower (428 -> 440 us).
        if constexpr (!FINAL) __builtin_amdgcn_sched_barrier(0);
        if constexpr (V == 0) {
            // the plain path, exponential-Euler with Delta as given
            const float u = dv * xv;
            if constexpr (FINAL) {
                float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float ab = exp2_fast(dv * A2[n]);
                    h[n] = __builtin_fmaf(ab, h[n], u * Bt.at(n));
                    if (n & 1) y1 = __builtin_fmaf(Ct.at(n), h[n], y1);
                    else y0 = __builtin_fmaf(Ct.at(n), h[n], y0);
                }
                float v = y0 + y1;
                if constexpr (SINK) {
                    lsink[k * 64 + (threadIdx.x & 63)] = v;
                } else {
                    if constexpr (HAS_D) v = __builtin_fmaf(Dv, xv, v);
                    if constexpr (HAS_Z) v *= silu(zv);
                    store_io<BF16>(ry, yoff, (uint32_t)t * ystride, v);
                }
            } else {
                sumd += dv;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float ab = exp2_fast(dv * A2[n]);
                    h[n] = __builtin_fmaf(ab, h[n], u * Bt.at(n));
                }
            }
            return;
        }
        float y0 = 0.0f, y1 = 0.0f;
        if constexpr (V == 2) {
            // the blended form only when some lane of the wave has a small |z| this step
            if (__builtin_amdgcn_ballot_w64(fabsf(dv) * vl.amin2 < kZohSmall2) != 0)
                states<1>(A2, h, dv, xv, Bt, Ct, vl, y0, y1);
            else
                states<0>(A2, h, dv, xv, Bt, Ct, vl, y0, y1);
        } else {
            states<0>(A2, h, dv, xv, Bt, Ct, vl, y0, y1);  // V = 1: exponential-Euler
        }
        if constexpr (FINAL) {
            float v = y0 + y1;
            if constexpr (SINK) {
                lsink[k * 64 + (threadIdx.x & 63)] = v;
            } else {
                if constexpr (HAS_D) v = __builtin_fmaf(Dv, xv, v);
                if constexpr (HAS_Z) v *= silu(zv);
                store_io<BF16>(ry, yoff, (uint32_t)t * ystride, v);
            }
        } else {
            sumd += dv;
        }
    }

    // the whole segment from state h: full blocks of kP steps with a
    // static ring slot per step, then the tail straight from the ring.
    __device__ __forceinline__ void run(const float (&A2)[N], float (&h)[N], float Dv, float& sumd,
                                        const VarLane<N, V>& vl) {
        int t = 0;
        for (; t + kP <= len; t += kP) {
#pragma unroll
            for (int k = 0; k < kP; ++k) step<true>(t + k, k, A2, h, Dv, sumd, vl);
        }
#pragma unroll
        for (int k = 0; k < kP - 1; ++k)
            if (t + k < len) step<false>(t + k, k, A2, h, Dv, sumd, vl);
    }
};

template <int N, bool BF16, int V = 0>
__global__ void __launch_bounds__(64 * SSM_SCAN_MAX_GROUP)
segment_aggregate(ScanArgs a, Geom g) {
    extern __shared__ float lds[];
    const int W = g.W;
    // the wave index is uniform across the wave: say so, so that everything derived
    // from it (segment, descriptors, offsets) lives in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = blockIdx.x, b = blockIdx.z;
    const int D = a.D, NT = a.N;
    const int nch = NT / N, nc = blockIdx.y % nch, n0 = nc * N;  // state chunk of this block
    const int d = (blockIdx.y / nch) * 64 + lane;
    const int dc = d < D ? d : D - 1;
    const int s = grp * W + wave;
    const int t0 = s * g.Ls;
    const int len = s < g.S ? min(g.Ls, a.L - t0) : 0;

    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[(size_t)dc * NT + n0 + n] * kLog2e;
        h[n] = 0.0f;
    }
    float sumd = 0.0f;
    VarLane<N, V> vl;
    var_lane_init<N, V>(vl, a, dc, n0);
    if (len > 0) {
        Segment<N, BF16, false, false, false, V> seg(a, b, dc, t0, len, n0);
        seg.run(A2, h, 0.0f, sumd, vl);
    }
    // LDS: H[w][n][lane], SD[w][lane]; a segment past L is the identity (sum 0, H 0).
    // A segment's decay exp2(A2 sum Delta) is recomputed by the waves that need it
    // (the same lane holds the same channel's A), so only H and the sum go through
    // LDS: less LDS per workgroup, more workgroups per CU.
    float* sH = lds;
    float* sS = sH + W * N * 64;
#pragma unroll
    for (int n = 0; n < N; ++n) sH[(wave * N + n) * 64 + lane] = h[n];
    sS[wave * 64 + lane] = sumd;
    __syncthreads();

    float E[N];
#pragma unroll
    for (int n = 0; n < N; ++n) E[n] = 0.0f;
    float cs = 0.0f;
    for (int j = 0; j < wave; ++j) {
        const float sj = sS[j * 64 + lane];
#pragma unroll
        for (int n = 0; n < N; ++n)
            E[n] = __builtin_fmaf(exp2_fast(A2[n] * sj), E[n], sH[(j * N + n) * 64 + lane]);
        cs += sj;
    }
    if (d >= D || s >= g.S) return;
    const WsLayout wl = ws_layout(a.B, D, NT, g.S, g.G);
    float* ws = static_cast<float*>(a.ws);
    if (wave > 0) {  // the first segment of a group starts from the group's own entering state
        float* Ep = ws + wl.E + (((size_t)b * g.S + s) * NT + n0) * D + d;
#pragma unroll
        for (int n = 0; n < N; ++n) Ep[(size_t)n * D] = E[n];
        if (nc == 0) ws[wl.CS + ((size_t)b * g.S + s) * D + d] = cs;
    }
    // the group's own aggregate, needed by later groups
    const bool last_in_group = (wave == W - 1) || (s == g.S - 1);
    if (last_in_group && grp < g.G - 1) {
        float* GH = ws + wl.GH + (((size_t)b * (g.G - 1) + grp) * NT + n0) * D + d;
        float* GP = ws + wl.GP + (((size_t)b * (g.G - 1) + grp) * NT + n0) * D + d;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            GH[(size_t)n * D] = __builtin_fmaf(exp2_fast(A2[n] * sumd), E[n], h[n]);
            GP[(size_t)n * D] = exp2_fast(A2[n] * (cs + sumd));
        }
    }
}

// state entering each group: carry(0) = h0, carry(g+1) = GP_g carry(g) + GH_g,
// written over GH_g. Workgroup of 64 channels x 4 quarters of the G-1 groups:
// each thread composes its quarter's affine maps, the quarters' composites are
// chained in LDS, then each thread walks its quarter again from its entering state.
__global__ void __launch_bounds__(256)
group_carry(const float* __restrict__ h0, float* ws, int B, int D, int N, Geom g) {
    __shared__ float sP[4][64], sH[4][64];
    const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int d = blockIdx.x * 64 + lane, n = blockIdx.y, b = blockIdx.z;
    const int dc = d < D ? d : D - 1;
    const WsLayout wl = ws_layout(B, D, N, g.S, g.G);
    const size_t st = (size_t)N * D;
    float* GH = ws + wl.GH + (size_t)b * (g.G - 1) * st + (size_t)n * D + dc;
    const float* GP = ws + wl.GP + (size_t)b * (g.G - 1) * st + (size_t)n * D + dc;
    const int steps = g.G - 1, per = (steps + 3) / 4;
    const int k0 = min(q * per, steps), k1 = min(k0 + per, steps);
    constexpr int U = 16;  // a quarter of at most U groups stays in registers
    float p[U], v[U];
    float cp = 1.0f, ch = 0.0f;
    const bool in_regs = per <= U;  // uniform
    for (int k = k0; k < k1; k += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = min(k + u, k1 - 1);
            p[u] = GP[kk * st];
            v[u] = GH[kk * st];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k + u < k1) {
                ch = __builtin_fmaf(p[u], ch, v[u]);
                cp *= p[u];
            }
        }
    }
    sP[q][lane] = cp;
    sH[q][lane] = ch;
    __syncthreads();
    float h = h0 ? h0[((size_t)b * D + dc) * N + n] : 0.0f;
    for (int j = 0; j < q; ++j) h = __builtin_fmaf(sP[j][lane], h, sH[j][lane]);
    if (d >= D) return;
    for (int k = k0; k < k1; k += U) {
        if (!in_regs) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kk = min(k + u, k1 - 1);
                p[u] = GP[kk * st];
                v[u] = GH[kk * st];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k + u < k1) {
                h = __builtin_fmaf(p[u], h, v[u]);
                GH[(k + u) * st] = h;
            }
        }
    }
}

template <int N, bool BF16, bool HAS_Z, bool HAS_D, int V = 0>
__global__ void __launch_bounds__(64 * SSM_SCAN_MAX_GROUP)
segment_final(ScanArgs a, Geom g) {
    const int W = g.W;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = blockIdx.x, b = blockIdx.z;
    const int D = a.D, NT = a.N;
    const int nch = NT / N, nc = blockIdx.y % nch, n0 = nc * N;  // state chunk of this block
    const int d = (blockIdx.y / nch) * 64 + lane;
    const int dc = d < D ? d : D - 1;
    const int s = grp * W + wave;
    const int t0 = s * g.Ls;
    if (s >= g.S) return;
    const int len = min(g.Ls, a.L - t0);
    const WsLayout wl = ws_layout(a.B, D, NT, g.S, g.G);
    const float* ws = static_cast<const float*>(a.ws);

    // every load that does not depend on the recurrence first: the segment's
    // first inputs, A, the state entering the group and the in-group prefix
    Segment<N, BF16, HAS_Z, HAS_D, true, V> seg(a, b, dc, t0, len, n0, d < D);
    float A2[N], hg[N], E[N];
    float cs = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = a.A[(size_t)dc * NT + n0 + n] * kLog2e;
    if (grp > 0) {
        const float* cp = ws + wl.GH + (((size_t)b * (g.G - 1) + grp - 1) * NT + n0) * D + dc;
#pragma unroll
        for (int n = 0; n < N; ++n) hg[n] = cp[(size_t)n * D];
    } else if (a.h0 != nullptr) {
        const float* hp = a.h0 + ((size_t)b * D + dc) * NT + n0;
#pragma unroll
        for (int n = 0; n < N; ++n) hg[n] = hp[n];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) hg[n] = 0.0f;
    }
    if (wave > 0) {
        cs = ws[wl.CS + ((size_t)b * g.S + s) * D + dc];
        const float* Ep = ws + wl.E + (((size_t)b * g.S + s) * NT + n0) * D + dc;
#pragma unroll
        for (int n = 0; n < N; ++n) E[n] = Ep[(size_t)n * D];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) E[n] = 0.0f;
    }
    float h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = __builtin_fmaf(exp2_fast(A2[n] * cs), hg[n], E[n]);
    // the variants run with HAS_D and D = 0 when the skip is absent
    const float Dv = (HAS_D && (V == 0 || a.Dskip != nullptr)) ? a.Dskip[dc] : 0.0f;
    float unused = 0.0f;
    VarLane<N, V> vl;
    var_lane_init<N, V>(vl, a, dc, n0);
    seg.run(A2, h, Dv, unused, vl);
    if (d < D && s == g.S - 1 && a.h_final != nullptr) {
        float* hp = a.h_final + ((size_t)b * D + d) * NT + n0;
#pragma unroll
        for (int n = 0; n < N; ++n) hp[n] = h[n];
    }
}

// A short chain (2 .. kFusedSegs segments, N <= 32): one workgroup of one wave per
// segment runs the whole call. Each wave runs its segment from a zero state, the
// waves meet in LDS for the exclusive prefix of the earlier segments (their end
// states and sums of Delta; decays recomputed from the sums), and each wave runs its
// segment again from its entering state, writing y. One launch, no workspace.
constexpr int kFusedSegs = 8;

template <int N, bool BF16, bool HAS_Z, bool HAS_D, int V = 0>
__global__ void __launch_bounds__(64 * kFusedSegs)
segment_fused(ScanArgs a, Geom g) {
    extern __shared__ float lds[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int b = blockIdx.z, D = a.D;
    const int d = blockIdx.y * 64 + lane;
    const int dc = d < D ? d : D - 1;
    const int s = wave;
    const int t0 = s * g.Ls;
    const int len = s < g.S ? min(g.Ls, a.L - t0) : 0;

    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[(size_t)dc * N + n] * kLog2e;
        h[n] = 0.0f;
    }
    VarLane<N, V> vl;
    var_lane_init<N, V>(vl, a, dc, 0);
    float sumd = 0.0f;
    if (len > 0) {
        Segment<N, BF16, false, false, false, V> seg(a, b, dc, t0, len, 0);
        seg.run(A2, h, 0.0f, sumd, vl);
    }
    float* sH = lds;
    float* sS = sH + kFusedSegs * N * 64;
#pragma unroll
    for (int n = 0; n < N; ++n) sH[(wave * N + n) * 64 + lane] = h[n];
    sS[wave * 64 + lane] = sumd;
    __syncthreads();
    if (len == 0) return;
    // entering state: exp2(A2 * prefix sum Delta) h0 + the earlier segments' composite
    float E[N];
#pragma unroll
    for (int n = 0; n < N; ++n) E[n] = 0.0f;
    float cs = 0.0f;
    for (int j = 0; j < wave; ++j) {
        const float sj = sS[j * 64 + lane];
#pragma unroll
        for (int n = 0; n < N; ++n)
            E[n] = __builtin_fmaf(exp2_fast(A2[n] * sj), E[n], sH[(j * N + n) * 64 + lane]);
        cs += sj;
    }
    if (a.h0 != nullptr) {
        const float* hp = a.h0 + ((size_t)b * D + dc) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = __builtin_fmaf(exp2_fast(A2[n] * cs), hp[n], E[n]);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = E[n];
    }
    const float Dv = (HAS_D && (V == 0 || a.Dskip != nullptr)) ? a.Dskip[dc] : 0.0f;
    float unused = 0.0f;
    Segment<N, BF16, HAS_Z, HAS_D, true, V> seg(a, b, dc, t0, len, 0, d < D);
    seg.run(A2, h, Dv, unused, vl);
    if (d < D && s == g.S - 1 && a.h_final != nullptr) {
        float* hp = a.h_final + ((size_t)b * D + d) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) hp[n] = h[n];
    }
}

// A chain of 2 .. kFusedSegs segments with a single chunk of states runs as one
// launch when its waves get a SIMD each (at most four segments) or when the call has
// enough chains to put two or more waves on every SIMD anyway: with few chains, five to
// eight segments in one workgroup would share SIMDs that the separate launches spread
// over two CUs (B1 L256 D64: 24 -> 26 us), while a batch of short sequences gains
// (B64 L256 D1536: 178 -> 131-153 us).
inline bool fused_call(const Geom& g, int B, int D, int N) {
    if (g.S <= 1 || g.S > kFusedSegs || n_chunks(N) != 1) return false;
    const long waves = (long)B * ((D + 63) / 64) * g.S;
    return g.S <= 4 || waves >= 2048;
}

// N >= 64: one workgroup per (segment, 64 channels, batch, group of up to
// kSinkChunks state chunks) holds those chunks of the segment, one wave each. Every
// kPrefetch steps the waves leave their partial C . h sums in LDS (two slots,
// alternating), meet at a barrier, and the workgroup adds them in chunk order into
// one fp32 sum per (t, channel). FUSE (one chunk group, N <= 128): the workgroup
// holds every state chunk, so it finishes y itself (D x, the gate, the rounding);
// otherwise the sums go to the group's plane of YP and combine_partials adds the
// planes, D x and the gate.
constexpr int kSinkChunks = 8;
inline int sink_planes(int N) { return std::max(1, n_chunks(N) / kSinkChunks); }
static_assert(64 / kChunkN >= kPrefetch, "a fused sink needs a wave per step of the ring");

template <bool BF16, int V = 0, bool FUSE = false>
__global__ void __launch_bounds__(64 * kSinkChunks)
segment_final_sink(ScanArgs a, Geom g) {
    extern __shared__ float lds[];
    constexpr int N = kChunkN;
    const int nch = blockDim.x >> 6;             // chunks in this workgroup
    const int ngrp = (a.N / N) / nch;            // chunk groups (planes of YP)
    const int cg = blockIdx.y % ngrp, dblk = blockIdx.y / ngrp;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int nc = cg * nch + wave;
    const int n0 = nc * N;
    const int s = blockIdx.x, b = blockIdx.z;
    const int D = a.D, NT = a.N;
    const int d = dblk * 64 + lane;
    const int dc = d < D ? d : D - 1;
    const int grp = s / g.W, win = s % g.W;
    const int t0 = s * g.Ls;
    const int len = min(g.Ls, a.L - t0);
    const WsLayout wl = ws_layout(a.B, D, NT, g.S, g.G);
    const float* ws = static_cast<const float*>(a.ws);
    float* yp = FUSE ? nullptr : static_cast<float*>(a.ws) + wl.YP + (size_t)cg * a.B * a.L * D;

    Segment<N, BF16, false, false, true, V, true> seg(a, b, dc, t0, len, n0, d < D);
    float A2[N], hg[N], E[N];
    float cs = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = a.A[(size_t)dc * NT + n0 + n] * kLog2e;
    if (grp > 0) {
        const float* cp = ws + wl.GH + (((size_t)b * (g.G - 1) + grp - 1) * NT + n0) * D + dc;
#pragma unroll
        for (int n = 0; n < N; ++n) hg[n] = cp[(size_t)n * D];
    } else if (a.h0 != nullptr) {
        const float* hp = a.h0 + ((size_t)b * D + dc) * NT + n0;
#pragma unroll
        for (int n = 0; n < N; ++n) hg[n] = hp[n];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) hg[n] = 0.0f;
    }
    if (win > 0) {
        cs = ws[wl.CS + ((size_t)b * g.S + s) * D + dc];
        const float* Ep = ws + wl.E + (((size_t)b * g.S + s) * NT + n0) * D + dc;
#pragma unroll
        for (int n = 0; n < N; ++n) E[n] = Ep[(size_t)n * D];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) E[n] = 0.0f;
    }
    float h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = __builtin_fmaf(exp2_fast(A2[n] * cs), hg[n], E[n]);
    float unused = 0.0f;
    VarLane<N, V> vl;
    var_lane_init<N, V>(vl, a, dc, n0);
    // FUSE: wave w finishes step tb + w of its lane's channel; its x and z are
    // loaded when the block of steps starts, so the loads overlap the block.
    const bool has_d = FUSE && a.Dskip != nullptr, has_z = FUSE && a.z != nullptr;
    const float Dv = has_d ? a.Dskip[dc] : 0.0f;
    const size_t row0 = (size_t)b * a.L + t0;
    float xr = 0.0f, zr = 0.0f;
    auto fetch_xz = [&](int tb) {
        const size_t i = (row0 + min(tb + wave, len - 1)) * D + dc;
        if (has_d) xr = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.x)[i]) : static_cast<const float*>(a.x)[i];
        if (has_z) zr = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.z)[i]) : static_cast<const float*>(a.z)[i];
    };
    // the sums of the steps [tb, tb + cnt) from LDS slot `slot`, in chunk order
    auto reduce = [&](int slot, int tb, int cnt) {
        const float* base = lds + (size_t)slot * nch * kPrefetch * 64;
        if constexpr (FUSE) {
            if (wave < cnt) {
                float v = 0.0f;
                for (int c = 0; c < nch; ++c) v += base[(c * kPrefetch + wave) * 64 + lane];
                if (has_d) v = __builtin_fmaf(Dv, xr, v);
                if (has_z) v *= silu(zr);
                const size_t i = (row0 + tb + wave) * D + d;
                if (d < D) {
                    if constexpr (BF16) static_cast<uint16_t*>(a.y)[i] = f32_to_bf16(v);
                    else static_cast<float*>(a.y)[i] = v;
                }
            }
        } else {
            for (int o = threadIdx.x; o < cnt * 64; o += nch * 64) {
                const int k = o >> 6, l = o & 63, dd = dblk * 64 + l;
                float v = 0.0f;
                for (int c = 0; c < nch; ++c) v += base[(c * kPrefetch + k) * 64 + l];
                if (dd < D) yp[(row0 + tb + k) * D + dd] = v;
            }
        }
    };
    int t = 0, j = 0;
    for (; t + kPrefetch <= len; t += kPrefetch, ++j) {
        seg.lsink = lds + ((size_t)(j & 1) * nch + wave) * kPrefetch * 64;
        if constexpr (FUSE) fetch_xz(t);
#pragma unroll
        for (int k = 0; k < kPrefetch; ++k) seg.template step<true>(t + k, k, A2, h, 0.0f, unused, vl);
        __syncthreads();
        reduce(j & 1, t, kPrefetch);
    }
    if (t < len) {
        seg.lsink = lds + ((size_t)(j & 1) * nch + wave) * kPrefetch * 64;
        if constexpr (FUSE) fetch_xz(t);
#pragma unroll
        for (int k = 0; k < kPrefetch - 1; ++k)
            if (t + k < len) seg.template step<false>(t + k, k, A2, h, 0.0f, unused, vl);
        __syncthreads();
        reduce(j & 1, t, len - t);
    }
    if (d < D && s == g.S - 1 && a.h_final != nullptr) {
        float* hp = a.h_final + ((size_t)b * D + d) * NT + n0;
#pragma unroll
        for (int n = 0; n < N; ++n) hp[n] = h[n];
    }
}

// L == 0: the final state is the initial state.
__global__ void copy_state(const float* __restrict__ h0, float* __restrict__ out, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

// N >= 64: y = (C . h summed over the state chunks + D x) silu(z), one thread per
// (b, t, d); the nch planes of sums are added in plane order.
template <bool BF16, bool HAS_Z, bool HAS_D>
__global__ void __launch_bounds__(256)
combine_partials(ScanArgs a, const float* __restrict__ yp, int nch) {
    const size_t tot = (size_t)a.B * a.L * a.D;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= tot) return;
    // eight chunks' partials loaded before any is added (added in chunk order)
    float v = 0.0f;
    for (int c0 = 0; c0 < nch; c0 += 8) {
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = yp[(size_t)min(c0 + j, nch - 1) * tot + i];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (c0 + j < nch) v += t[j];
    }
    if constexpr (HAS_D) {
        const float xv = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.x)[i]) : static_cast<const float*>(a.x)[i];
        v = __builtin_fmaf(a.Dskip[i % a.D], xv, v);
    }
    if constexpr (HAS_Z) {
        const float zv = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.z)[i]) : static_cast<const float*>(a.z)[i];
        v *= silu(zv);
    }
    if constexpr (BF16) static_cast<uint16_t*>(a.y)[i] = f32_to_bf16(v);
    else static_cast<float*>(a.y)[i] = v;
}

// N >= 64, after the aggregate and carry passes: the state chunks' final pass,
// finishing y itself when one workgroup holds every chunk, else into the planes
// of partial sums, then their sum with D x and the gate.
template <bool BF16, int V>
void launch_sink(const ScanArgs& a, const Geom& g, hipStream_t st) {
    const int nch = a.N / kChunkN;
    const int planes = sink_planes(a.N), cpw = nch / planes;
    const dim3 sgrid((unsigned)g.S, (unsigned)(((a.D + 63) / 64) * planes), (unsigned)a.B);
    const size_t lds_sink = (size_t)2 * cpw * kPrefetch * 64 * sizeof(float);
    if (planes == 1) {
        launch((segment_final_sink<BF16, V, true>), sgrid, dim3(64 * cpw), (uint32_t)lds_sink, st, a, g);
        return;
    }
    launch((segment_final_sink<BF16, V>), sgrid, dim3(64 * cpw), (uint32_t)lds_sink, st, a, g);
    const float* yp = static_cast<const float*>(a.ws) + ws_layout(a.B, a.D, a.N, g.S, g.G).YP;
    const size_t tot = (size_t)a.B * a.L * a.D;
    const dim3 cg((unsigned)((tot + 255) / 256));
    const bool hz = a.z != nullptr, hd = a.Dskip != nullptr;
    if (hz && hd) launch((combine_partials<BF16, true, true>), cg, dim3(256), 0, st, a, yp, planes);
    else if (hz) launch((combine_partials<BF16, true, false>), cg, dim3(256), 0, st, a, yp, planes);
    else if (hd) launch((combine_partials<BF16, false, true>), cg, dim3(256), 0, st, a, yp, planes);
    else launch((combine_partials<BF16, false, false>), cg, dim3(256), 0, st, a, yp, planes);
}

// N: states per lane (a.N itself when a.N <= 32, else the chunk of kChunkN).
// V: the discretisation (0 plain; 1, 2 the variants, which run the final pass
// with HAS_D and D = 0 when the skip is absent: exact, y + 0 x = y).
template <int N, bool BF16, int V = 0>
hipError_t launch_n(const ScanArgs& a, hipStream_t st) {
    const Geom g = geom(a.B, a.L, a.D, a.N);
    if (a.L == 0) {
        if (a.h_final) {
            const size_t n = (size_t)a.B * a.D * a.N;
            launch(copy_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.h0, a.h_final, n);
        }
        return hipGetLastError();
    }
    const int nch = a.N / N;
    const bool hz = a.z != nullptr, hd = a.Dskip != nullptr;
    if (fused_call(g, a.B, a.D, a.N)) {
        const dim3 fgrid(1, (a.D + 63) / 64, a.B), fblock(64 * g.S);
        const size_t lds_f = (size_t)kFusedSegs * (N + 1) * 64 * sizeof(float);
        if constexpr (V != 0) {
            if (hz) launch((segment_fused<N, BF16, true, true, V>), fgrid, fblock, lds_f, st, a, g);
            else launch((segment_fused<N, BF16, false, true, V>), fgrid, fblock, lds_f, st, a, g);
        } else {
            if (hz && hd) launch((segment_fused<N, BF16, true, true>), fgrid, fblock, lds_f, st, a, g);
            else if (hz) launch((segment_fused<N, BF16, true, false>), fgrid, fblock, lds_f, st, a, g);
            else if (hd) launch((segment_fused<N, BF16, false, true>), fgrid, fblock, lds_f, st, a, g);
            else launch((segment_fused<N, BF16, false, false>), fgrid, fblock, lds_f, st, a, g);
        }
        return hipGetLastError();
    }
    const dim3 grid(g.G, ((a.D + 63) / 64) * nch, a.B);
    const dim3 block(64 * g.W);
    const size_t lds_agg = (size_t)g.W * (N + 1) * 64 * sizeof(float);
    if (g.S > 1) launch((segment_aggregate<N, BF16, V>), grid, block, lds_agg, st, a, g);
    if (g.G > 1) {
        launch(group_carry, dim3((unsigned)((a.D + 63) / 64), (unsigned)a.N, (unsigned)a.B), dim3(256), 0, st,
               a.h0, static_cast<float*>(a.ws), a.B, a.D, a.N, g);
    }
    if (nch > 1) {
        launch_sink<BF16, V>(a, g, st);
        return hipGetLastError();
    }
    if constexpr (V != 0) {
        if (hz) launch((segment_final<N, BF16, true, true, V>), grid, block, 0, st, a, g);
        else launch((segment_final<N, BF16, false, true, V>), grid, block, 0, st, a, g);
    } else {
        if (hz && hd) launch((segment_final<N, BF16, true, true>), grid, block, 0, st, a, g);
        else if (hz) launch((segment_final<N, BF16, true, false>), grid, block, 0, st, a, g);
        else if (hd) launch((segment_final<N, BF16, false, true>), grid, block, 0, st, a, g);
        else launch((segment_final<N, BF16, false, false>), grid, block, 0, st, a, g);
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const ScanArgs& a, hipStream_t st) {
    switch (a.N) {
        case 4: return launch_n<4, BF16>(a, st);
        case 8: return launch_n<8, BF16>(a, st);
        case 16: return launch_n<16, BF16>(a, st);
        case 32: return launch_n<32, BF16>(a, st);
        case 64:
        case 128:
        case 256: return launch_n<kChunkN, BF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace ssm
