// Mamba-2 SSD chunked scan on gfx950 ("Efficient Sequence Modeling: From S4 to
// Mamba-3", section 03, mamba2_minimal.py: a scalar A per head turns the
// recurrence into chunked decayed-attention matmuls with a carried (N, P) state;
// Dao & Gu 2024, "Transformers are SSMs").
//
// Per head h, with a_t = exp(Delta_t A_h) and, inside a chunk, the inclusive
// prefix s_i = sum_{k<=i} Delta_k A_h (kept in log2 units, accumulated in fp64
// and rounded once), the chunk's outputs are
//   y_i = exp(s_i) C_i . H_in  +  sum_{j<=i} (C_i . B_j) exp(s_i - s_j) Delta_j x_j
// and the state after it is H_out = exp(s_last) H_in + sum_j exp(s_last - s_j) Delta_j B_j (x) x_j.
//
// Kernels (one workgroup of 8 waves per (batch, head, super-chunk); a
// super-chunk is a run of consecutive chunks walked in order):
//   ssd_super_state  every super-chunk but the last: its aggregate state from a
//                    zero start, and its total log2 decay;
//   ssd_chunk_scan   folds the aggregates of earlier super-chunks into the state
//                    entering its own, then for every chunk: Y_off = diag(e^s) C H,
//                    G^T = B C^T, M = G o decay o Delta (causal), Y_diag = M X,
//                    y = (Y_off + Y_diag + D x) silu(z), then the chunk state
//                    S = (w o X)^T B and H <- e^{s_last} H + S.
// The fp32 state H^T (P x N) lives in registers, each wave owning the 16x16 tiles
// it accumulates S into; after every update its bf16 high part and bf16
// remainder are written to LDS, where they are the operands of Y_off.
// Matrix cores: v_mfma_f32_16x16x32_bf16 throughout. Operands stored in bf16
// (B, C, x) enter exactly; operands formed in fp32 (H, M, w o x) enter as a bf16
// high part plus a bf16 remainder, i.e. two MFMAs, which keeps about 16
// significant bits (one bf16 rounding would cost ~1e-3 relative error).
// x and B rows of a chunk are staged in LDS with 16-byte copies (loaded one chunk
// ahead into registers); where a product contracts over time, its operand is read
// with the LDS transpose read (ds_read_b64_tr_b16), which hands each lane four
// consecutive time steps of one column.
// Below the diagonal, exp2(s_i - s_j) = exp2(s_i - s_r) exp2(s_r - s_j) with r the
// last step of j's 32-step block: one exp per row and a per-column factor staged
// once per chunk (both factors <= 1, so neither can overflow).
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTargetBlocks = 768;  // workgroups of the scan kernel
constexpr int kP = 64;              // head dim handled
constexpr int kXS = kP + 16;        // LDS row stride (elements) of x rows
constexpr int kPad = 16;            // LDS row padding (elements) of B rows
constexpr int kHPad = 8;            // LDS row padding (elements) of the bf16 state rows

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v = hi + lo with hi the truncation of v to bf16 (exact) and lo = bf16(v - hi)
__device__ __forceinline__ void split8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t u = __float_as_uint(v[e]) & 0xffff0000u;
        hi[e] = __builtin_bit_cast(__bf16, (u16)(u >> 16));
        lo[e] = (__bf16)(v[e] - __uint_as_float(u));
    }
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const void* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Transposed operand read from a row-major [k][m] bf16 array in LDS (row stride
// `rs` elements): lane i of each 16-lane group receives rows k0 .. k0+3 of column
// m0 + i. Each lane of the group points at row k0 + i/4, columns m0 + 4(i%4) ...+3.
__device__ __forceinline__ bf16x4 ld_tr4(const u16* base, int rs, int k0, int m0) {
    const int i = threadIdx.x & 15;
    const u16* p = base + (k0 + (i >> 2)) * rs + m0 + 4 * (i & 3);
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

struct SsdGeom {
    int Q;    // chunk length
    int C;    // chunks per sequence
    int cps;  // chunks per super-chunk
    int K;    // super-chunks per sequence
};

SsdGeom ssd_geom(int B, int L, int H, int Q) {
    SsdGeom g;
    g.Q = Q;
    g.C = L > 0 ? (L + Q - 1) / Q : 0;
    const long bh = (long)B * H;
    long K = (kTargetBlocks + bh - 1) / bh;
    K = std::max<long>(1, std::min<long>(K, g.C));
    g.cps = g.C > 0 ? (int)((g.C + K - 1) / K) : 1;
    g.K = g.C > 0 ? (g.C + g.cps - 1) / g.cps : 0;
    return g;
}

// LDS layout (bytes), per workgroup
struct Smem {
    int xs, bs, hh, hl, s2, dt, w, cf, red, total;
};

template <int N>
__host__ __device__ inline Smem smem_layout(int Q) {
    Smem s;
    s.xs = 0;                              // bf16 [Q][kXS]       x rows of the chunk
    s.bs = s.xs + Q * kXS * 2;             // bf16 [Q][N+kPad]    B rows of the chunk
    s.hh = s.bs + Q * (N + kPad) * 2;      // bf16 [P][N+kHPad]   state H^T, high part
    s.hl = s.hh + kP * (N + kHPad) * 2;    // bf16 [P][N+kHPad]   state H^T, remainder
    s.s2 = s.hl + kP * (N + kHPad) * 2;    // f32  [Q]   inclusive log2-decay prefix
    s.dt = s.s2 + Q * 4;                   // f32  [Q]   Delta
    s.w = s.dt + Q * 4;                    // f32  [Q]   exp2(s_last - s_t) Delta_t
    s.cf = s.w + Q * 4;                    // f32  [Q]   exp2(s_r - s_t) Delta_t, r = t | 31
    s.red = s.cf + Q * 4;                  // f32  [4]   broadcast slot (s_last)
    s.total = s.red + 16;
    return s;
}

// workspace (floats): Hagg [B][H][K-1][P][N], Lam [B][H][K-1]
__host__ __device__ inline size_t ws_hagg(int B, int H, int K, int N) { return (size_t)B * H * (K - 1) * kP * N; }

// Rows of x and B of one chunk held in registers between the global load and the
// LDS store (so the next chunk's loads overlap the current chunk's work).
template <int N>
struct ChunkRows {
    static constexpr int XQ = 256 * (kP / 8) / kThreads;   // 16-byte pieces per thread, Q = 256
    static constexpr int BQ = 256 * (N / 8) / kThreads;
    uint4 xv[XQ];
    uint4 bv[BQ];
    float dv[4];
};

template <int N>
__device__ __forceinline__ void load_x_rows(const SsdArgs& a, int b, int h, int t0, int len, ChunkRows<N>& cr) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int k = 0; k < ChunkRows<N>::XQ; ++k) {
        const int q = tid + k * kThreads;
        const int r = q / (kP / 8), c8 = (q % (kP / 8)) * 8;
        cr.xv[k] = make_uint4(0, 0, 0, 0);
        if (r < len)
            cr.xv[k] = *reinterpret_cast<const uint4*>(static_cast<const u16*>(a.x) +
                                                       (((size_t)b * a.L + t0 + r) * a.H + h) * kP + c8);
    }
    if (wave == 0) {
        const u16* dp = static_cast<const u16*>(a.delta);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = lane * 4 + k;
            cr.dv[k] = (t < len) ? bf16_to_f32(dp[((size_t)b * a.L + t0 + t) * a.H + h]) : 0.0f;
        }
    }
}

template <int N>
__device__ __forceinline__ void load_b_rows(const SsdArgs& a, int b, int t0, int len, ChunkRows<N>& cr) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < ChunkRows<N>::BQ; ++k) {
        const int q = tid + k * kThreads;
        const int r = q / (N / 8), c8 = (q % (N / 8)) * 8;
        cr.bv[k] = make_uint4(0, 0, 0, 0);
        if (r < len)
            cr.bv[k] = *reinterpret_cast<const uint4*>(static_cast<const u16*>(a.Bm) + ((size_t)b * a.L + t0 + r) * N + c8);
    }
}

// Write a chunk's rows into LDS and (wave 0) its decay prefix, weights and column factors.
template <int N>
__device__ __forceinline__ void store_rows(char* lds, const Smem& sm, int Q, int len, float A2, const ChunkRows<N>& cr) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    u16* xs = reinterpret_cast<u16*>(lds + sm.xs);
    u16* bs = reinterpret_cast<u16*>(lds + sm.bs);
#pragma unroll
    for (int k = 0; k < ChunkRows<N>::XQ; ++k) {
        const int q = tid + k * kThreads;
        const int r = q / (kP / 8), c8 = (q % (kP / 8)) * 8;
        if (r < Q) *reinterpret_cast<uint4*>(xs + r * kXS + c8) = cr.xv[k];
    }
#pragma unroll
    for (int k = 0; k < ChunkRows<N>::BQ; ++k) {
        const int q = tid + k * kThreads;
        const int r = q / (N / 8), c8 = (q % (N / 8)) * 8;
        if (r < Q) *reinterpret_cast<uint4*>(bs + r * (N + kPad) + c8) = cr.bv[k];
    }
    if (wave == 0) {
        float* s2 = reinterpret_cast<float*>(lds + sm.s2);
        float* dt = reinterpret_cast<float*>(lds + sm.dt);
        float* w = reinterpret_cast<float*>(lds + sm.w);
        float* cf = reinterpret_cast<float*>(lds + sm.cf);
        // 4 consecutive steps per lane (Q <= 256), fp64 prefix, then a wave-wide scan
        double loc[4], run = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            run += (double)(cr.dv[k] * A2);
            loc[k] = run;
        }
        double incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        const double excl = incl - run;
        float sv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = lane * 4 + k;
            sv[k] = (float)(excl + loc[k]);
            if (t >= len) sv[k] = 0.0f;
        }
        float sl;
        {
            const int ll = (len - 1) >> 2, kk = (len - 1) & 3;
            const float lk = kk == 0 ? sv[0] : kk == 1 ? sv[1] : kk == 2 ? sv[2] : sv[3];
            sl = __shfl(lk, ll, 64);
        }
        // end of each 32-step block (lanes 8m .. 8m+7 cover block m): held by lane 8m+7, element 3
        const float send = __shfl(sv[3], (lane & ~7) | 7, 64);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = lane * 4 + k;
            if (t < Q) {
                const float s = t < len ? sv[k] : sl;
                const float r = min(t | 31, len - 1) == t ? s : (((t | 31) < len) ? send : sl);
                s2[t] = s;
                dt[t] = cr.dv[k];
                w[t] = t < len ? exp2_fast(sl - s) * cr.dv[k] : 0.0f;
                cf[t] = t < len ? exp2_fast(r - s) * cr.dv[k] : 0.0f;
            }
        }
        if (lane == 0) reinterpret_cast<float*>(lds + sm.red)[0] = sl;
    }
}

// Chunk state S^T = (w o X)^T B on this wave's tiles: p-block pb = wave % 4 and
// n-blocks nb0 .. nb0 + NBW - 1. Lane holds S^T[p = pb*16 + 4g + r][n = nb*16 + l%16].
template <int N>
struct StateTiles {
    static constexpr int NBW = N / 32;  // n-blocks per wave (8 waves = 4 p-blocks x 2 halves)
    f32x4 acc[NBW];
};

template <int N>
__device__ __forceinline__ void chunk_state(const char* lds, const Smem& sm, int len, StateTiles<N>& st) {
    constexpr int NBW = StateTiles<N>::NBW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int pb = wave & 3, nb0 = (wave >> 2) * NBW;
    const u16* xs = reinterpret_cast<const u16*>(lds + sm.xs);
    const u16* bs = reinterpret_cast<const u16*>(lds + sm.bs);
    const float* w = reinterpret_cast<const float*>(lds + sm.w);
#pragma unroll
    for (int k = 0; k < NBW; ++k) st.acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kbn = (len + 31) >> 5;
    for (int kb = 0; kb < kbn; ++kb) {
        const int t = kb * 32 + 8 * g;
        const bf16x8 xv = cat(ld_tr4(xs, kXS, t, pb * 16), ld_tr4(xs, kXS, t + 4, pb * 16));
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + t);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + t + 4);
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = (float)xv[e] * w0[e];
            v[e + 4] = (float)xv[e + 4] * w1[e];
        }
        bf16x8 ahi, alo;
        split8(v, ahi, alo);
#pragma unroll
        for (int k = 0; k < NBW; ++k) {
            const int n0 = (nb0 + k) * 16;
            const bf16x8 bop = cat(ld_tr4(bs, N + kPad, t, n0), ld_tr4(bs, N + kPad, t + 4, n0));
            st.acc[k] = mfma(ahi, bop, st.acc[k]);
            st.acc[k] = mfma(alo, bop, st.acc[k]);
        }
    }
}

// The fp32 state on this wave's tiles (same layout as StateTiles).
template <int N>
struct State {
    f32x4 h[StateTiles<N>::NBW];
};

// H <- exp2(s_last) H + S (registers)
template <int N>
__device__ __forceinline__ void state_update(const char* lds, const Smem& sm, State<N>& hs, const StateTiles<N>& st) {
    const float decay = exp2_fast(reinterpret_cast<const float*>(lds + sm.red)[0]);
#pragma unroll
    for (int k = 0; k < StateTiles<N>::NBW; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) hs.h[k][r] = __builtin_fmaf(decay, hs.h[k][r], st.acc[k][r]);
}

// bf16 high part and remainder of this wave's state tiles into LDS
template <int N>
__device__ __forceinline__ void state_to_lds(char* lds, const Smem& sm, const State<N>& hs) {
    constexpr int NBW = StateTiles<N>::NBW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int pb = wave & 3, nb0 = (wave >> 2) * NBW;
    u16* hh = reinterpret_cast<u16*>(lds + sm.hh);
    u16* hl = reinterpret_cast<u16*>(lds + sm.hl);
#pragma unroll
    for (int k = 0; k < NBW; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = hs.h[k][r];
            const uint32_t u = __float_as_uint(v) & 0xffff0000u;
            const int off = (pb * 16 + 4 * g + r) * (N + kHPad) + (nb0 + k) * 16 + c;
            hh[off] = (u16)(u >> 16);
            hl[off] = f32_to_bf16(v - __uint_as_float(u));
        }
}

// Element (p, n) of this lane's state tiles, for k = n-block offset, r = row offset
template <int N>
__device__ __forceinline__ void tile_pn(int k, int r, int& p, int& n) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    p = (wave & 3) * 16 + 4 * g + r;
    n = ((wave >> 2) * StateTiles<N>::NBW + k) * 16 + c;
}

template <int N>
__global__ void __launch_bounds__(kThreads)
ssd_super_state(SsdArgs a, SsdGeom geo) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const Smem sm = smem_layout<N>(geo.Q);
    const int k = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const float A2 = a.A[h] * kLog2e;
    State<N> hs;
#pragma unroll
    for (int kk = 0; kk < StateTiles<N>::NBW; ++kk) hs.h[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
    double lam = 0.0;
    const int c0 = k * geo.cps, c1 = min(geo.C, c0 + geo.cps);
    ChunkRows<N> cr;
    load_x_rows<N>(a, b, h, c0 * geo.Q, min(geo.Q, a.L - c0 * geo.Q), cr);
    load_b_rows<N>(a, b, c0 * geo.Q, min(geo.Q, a.L - c0 * geo.Q), cr);
    for (int cc = c0; cc < c1; ++cc) {
        const int t0 = cc * geo.Q;
        const int len = min(geo.Q, a.L - t0);
        __syncthreads();  // previous chunk fully consumed
        store_rows<N>(lds, sm, geo.Q, len, A2, cr);
        __syncthreads();
        if (cc + 1 < c1) {
            const int ln = min(geo.Q, a.L - t0 - geo.Q);
            load_x_rows<N>(a, b, h, t0 + geo.Q, ln, cr);
            load_b_rows<N>(a, b, t0 + geo.Q, ln, cr);
        }
        StateTiles<N> st;
        chunk_state<N>(lds, sm, len, st);
        lam += (double)reinterpret_cast<const float*>(lds + sm.red)[0];
        state_update<N>(lds, sm, hs, st);
    }
    float* out = static_cast<float*>(a.ws) + (((size_t)b * a.H + h) * (geo.K - 1) + k) * kP * N;
#pragma unroll
    for (int kk = 0; kk < StateTiles<N>::NBW; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int p, n;
            tile_pn<N>(kk, r, p, n);
            out[p * N + n] = hs.h[kk][r];
        }
    if (threadIdx.x == 0) {
        float* lamp = static_cast<float*>(a.ws) + ws_hagg(a.B, a.H, geo.K, N);
        lamp[((size_t)b * a.H + h) * (geo.K - 1) + k] = (float)lam;
    }
}

// Outputs of one 16-row block I of a chunk, for NPB p-blocks starting at pb0.
template <int N, int NPB, bool HAS_Z, bool HAS_D>
__device__ __forceinline__ void chunk_rows(const SsdArgs& a, const char* lds, const Smem& sm, int b, int h,
                                           int t0, int len, int I, int pb0, const bf16x8 (&cop)[N / 32], float Dh) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const u16* xs = reinterpret_cast<const u16*>(lds + sm.xs);
    const u16* bs = reinterpret_cast<const u16*>(lds + sm.bs);
    const u16* hh = reinterpret_cast<const u16*>(lds + sm.hh);
    const u16* hl = reinterpret_cast<const u16*>(lds + sm.hl);
    const float* s2 = reinterpret_cast<const float*>(lds + sm.s2);
    const float* dt = reinterpret_cast<const float*>(lds + sm.dt);
    const float* cf = reinterpret_cast<const float*>(lds + sm.cf);
    const int ia = I * 16 + c;  // this lane's A-operand row
    f32x4 acc[NPB];
#pragma unroll
    for (int q = 0; q < NPB; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Y_off = C H: the state's bf16 high part and remainder (rows of H^T) are B operands
#pragma unroll
    for (int kb = 0; kb < N / 32; ++kb)
#pragma unroll
        for (int q = 0; q < NPB; ++q) {
            const int off = ((pb0 + q) * 16 + c) * (N + kHPad) + kb * 32 + 8 * g;
            acc[q] = mfma(cop[kb], ld_bf16x8(hh + off), acc[q]);
            acc[q] = mfma(cop[kb], ld_bf16x8(hl + off), acc[q]);
        }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float sc = exp2_fast(s2[I * 16 + 4 * g + r]);
#pragma unroll
        for (int q = 0; q < NPB; ++q) acc[q][r] *= sc;
    }
    // Y_diag = M X over 32-wide column blocks J up to the block's last row
    const float s2i = s2[ia];
    for (int J = 0; J * 32 <= I * 16 + 15; ++J) {
        f32x4 g0 = f32x4{0.f, 0.f, 0.f, 0.f}, g1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < N / 32; ++kb) {
            const bf16x8 b0 = ld_bf16x8(bs + (J * 32 + c) * (N + kPad) + kb * 32 + 8 * g);
            const bf16x8 b1 = ld_bf16x8(bs + (J * 32 + 16 + c) * (N + kPad) + kb * 32 + 8 * g);
            g0 = mfma(b0, cop[kb], g0);  // G^T[j][i]: lane holds G[ia][J*32 + 4g + r]
            g1 = mfma(b1, cop[kb], g1);  //            and G[ia][J*32 + 16 + 4g + r]
        }
        float m[8];
        if (J * 32 + 31 < I * 16) {
            // whole column block below this row block: row factor x column factor
            const float rowf = exp2_fast(s2i - s2[J * 32 + 31]);
            const f32x4 c0 = *reinterpret_cast<const f32x4*>(cf + J * 32 + 4 * g);
            const f32x4 c1 = *reinterpret_cast<const f32x4*>(cf + J * 32 + 16 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                m[e] = g0[e] * rowf * c0[e];
                m[e + 4] = g1[e] * rowf * c1[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = J * 32 + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
                const float gv = e < 4 ? g0[e] : g1[e - 4];
                const bool ok = (j <= ia) && (j < len);
                m[e] = ok ? gv * exp2_fast(s2i - s2[j]) * dt[j] : 0.0f;
            }
        }
        bf16x8 mhi, mlo;
        split8(m, mhi, mlo);
#pragma unroll
        for (int q = 0; q < NPB; ++q) {
            // x at the same (g, e) -> j mapping: two runs of 4 steps
            const bf16x8 xop = cat(ld_tr4(xs, kXS, J * 32 + 4 * g, (pb0 + q) * 16),
                                   ld_tr4(xs, kXS, J * 32 + 16 + 4 * g, (pb0 + q) * 16));
            acc[q] = mfma(mhi, xop, acc[q]);
            acc[q] = mfma(mlo, xop, acc[q]);
        }
    }
    // epilogue: rows i = I*16 + 4g + r, columns p = (pb0 + q)*16 + c
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = I * 16 + 4 * g + r;
        if (i >= len) continue;
        const size_t rowoff = (((size_t)b * a.L + t0 + i) * a.H + h) * kP;
#pragma unroll
        for (int q = 0; q < NPB; ++q) {
            const int p = (pb0 + q) * 16 + c;
            float v = acc[q][r];
            if constexpr (HAS_D) v = __builtin_fmaf(Dh, bf16_to_f32(xs[i * kXS + p]), v);
            if constexpr (HAS_Z) v *= silu(bf16_to_f32(static_cast<const u16*>(a.z)[rowoff + p]));
            static_cast<u16*>(a.y)[rowoff + p] = f32_to_bf16(v);
        }
    }
}

template <int N, bool HAS_Z, bool HAS_D>
__global__ void __launch_bounds__(kThreads)
ssd_chunk_scan(SsdArgs a, SsdGeom geo) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const Smem sm = smem_layout<N>(geo.Q);
    const int k = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const float A2 = a.A[h] * kLog2e;
    const float Dh = HAS_D ? a.Dskip[h] : 0.0f;
    const int c0 = k * geo.cps, c1 = min(geo.C, c0 + geo.cps);

    ChunkRows<N> cr;
    load_x_rows<N>(a, b, h, c0 * geo.Q, min(geo.Q, a.L - c0 * geo.Q), cr);
    load_b_rows<N>(a, b, c0 * geo.Q, min(geo.Q, a.L - c0 * geo.Q), cr);

    // state entering this super-chunk: h0 folded with the earlier aggregates
    State<N> hs;
    {
        const float* hagg = static_cast<const float*>(a.ws);
        const float* lamp = hagg + ws_hagg(a.B, a.H, geo.K, N);
#pragma unroll
        for (int kk = 0; kk < StateTiles<N>::NBW; ++kk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int p, n;
                tile_pn<N>(kk, r, p, n);
                hs.h[kk][r] = a.h0 ? a.h0[(((size_t)b * a.H + h) * N + n) * kP + p] : 0.0f;
            }
        for (int j = 0; j < k; ++j) {
            const size_t base = ((size_t)b * a.H + h) * (geo.K - 1) + j;
            const float dec = exp2_fast(lamp[base]);
#pragma unroll
            for (int kk = 0; kk < StateTiles<N>::NBW; ++kk)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int p, n;
                    tile_pn<N>(kk, r, p, n);
                    hs.h[kk][r] = __builtin_fmaf(dec, hs.h[kk][r], hagg[base * kP * N + p * N + n]);
                }
        }
        state_to_lds<N>(lds, sm, hs);
    }
    const bool last_super = (k == geo.K - 1);
    const u16* Cg = static_cast<const u16*>(a.Cm);
    // Work split of the output phase over the 8 waves, by the number R of 16-row blocks:
    //   R >= 8: wave w takes block w and, when R - 1 - w >= 8, block R - 1 - w too
    //           (pairs balance the causal work), all 4 p-blocks;
    //   R = 4:  wave w takes block w % 4 and 2 of the p-blocks;
    //   R = 2:  wave w takes block w % 2 and 1 p-block;
    //   R = 6:  waves 0..5 take one block each, all p-blocks.
    const int R = geo.Q / 16;
    int I0 = wave, I1 = -1, npb = 4, pb0 = 0;
    if (R >= 8) {
        if (R - 1 - wave >= 8) I1 = R - 1 - wave;
    } else if (R == 4) {
        I0 = wave & 3; npb = 2; pb0 = (wave >> 2) * 2;
    } else if (R == 2) {
        I0 = wave & 1; npb = 1; pb0 = wave >> 1;
    } else if (wave >= R) {
        I0 = -1;
    }
    for (int cc = c0; cc < c1; ++cc) {
        const int t0 = cc * geo.Q;
        const int len = min(geo.Q, a.L - t0);
        // C rows of this wave's blocks straight from global
        bf16x8 cop0[N / 32], cop1[N / 32];
#pragma unroll
        for (int kb = 0; kb < N / 32; ++kb) {
            const int i0 = I0 * 16 + c, i1 = I1 * 16 + c;
            cop0[kb] = (I0 >= 0 && i0 < len) ? ld_bf16x8(Cg + ((size_t)b * a.L + t0 + i0) * N + kb * 32 + 8 * g) : bf16x8{};
            cop1[kb] = (I1 >= 0 && i1 < len) ? ld_bf16x8(Cg + ((size_t)b * a.L + t0 + i1) * N + kb * 32 + 8 * g)
                                             : bf16x8{};
        }
        __syncthreads();  // previous chunk's LDS reads done, state copy written
        store_rows<N>(lds, sm, geo.Q, len, A2, cr);
        __syncthreads();
        // next chunk's x rows and Delta load during the output phase, its B rows after it
        const int ln = cc + 1 < c1 ? min(geo.Q, a.L - t0 - geo.Q) : 0;
        if (ln > 0) load_x_rows<N>(a, b, h, t0 + geo.Q, ln, cr);
        if (I0 >= 0 && I0 * 16 < len) {
            if (npb == 4) chunk_rows<N, 4, HAS_Z, HAS_D>(a, lds, sm, b, h, t0, len, I0, pb0, cop0, Dh);
            else if (npb == 2) chunk_rows<N, 2, HAS_Z, HAS_D>(a, lds, sm, b, h, t0, len, I0, pb0, cop0, Dh);
            else chunk_rows<N, 1, HAS_Z, HAS_D>(a, lds, sm, b, h, t0, len, I0, pb0, cop0, Dh);
        }
        if (I1 >= 0 && I1 * 16 < len) chunk_rows<N, 4, HAS_Z, HAS_D>(a, lds, sm, b, h, t0, len, I1, 0, cop1, Dh);
        if (ln > 0) load_b_rows<N>(a, b, t0 + geo.Q, ln, cr);
        // state after the chunk (not needed after the last chunk of a super-chunk,
        // except at the very end of the sequence for h_final)
        const bool need_state = (cc < c1 - 1) || (last_super && a.h_final != nullptr);
        if (need_state) {
            StateTiles<N> st;
            chunk_state<N>(lds, sm, len, st);
            state_update<N>(lds, sm, hs, st);
            __syncthreads();  // every wave has finished reading the state copy for Y_off
            if (cc < c1 - 1) state_to_lds<N>(lds, sm, hs);
        }
    }
    if (last_super && a.h_final != nullptr) {
#pragma unroll
        for (int kk = 0; kk < StateTiles<N>::NBW; ++kk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int p, n;
                tile_pn<N>(kk, r, p, n);
                a.h_final[(((size_t)b * a.H + h) * N + n) * kP + p] = hs.h[kk][r];
            }
    }
}

__global__ void copy_state_ssd(const float* __restrict__ h0, float* __restrict__ out, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

template <int N>
hipError_t launch_n(const SsdArgs& a, hipStream_t st) {
    if (a.L == 0) {
        if (a.h_final) {
            const size_t n = (size_t)a.B * a.H * N * a.P;
            profile_mark(st);
            hipLaunchKernelGGL(copy_state_ssd, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                               a.h0, a.h_final, n);
            profile_mark(st);
        }
        return hipGetLastError();
    }
    const SsdGeom geo = ssd_geom(a.B, a.L, a.H, a.Q);
    const Smem sm = smem_layout<N>(geo.Q);
    if (geo.K > 1) {
        profile_mark(st);
        hipLaunchKernelGGL((ssd_super_state<N>), dim3(geo.K - 1, a.H, a.B), dim3(kThreads), sm.total, st, a, geo);
    }
    const bool hz = a.z != nullptr, hd = a.Dskip != nullptr;
    const dim3 grid(geo.K, a.H, a.B);
    profile_mark(st);
    if (hz && hd) hipLaunchKernelGGL((ssd_chunk_scan<N, true, true>), grid, dim3(kThreads), sm.total, st, a, geo);
    else if (hz) hipLaunchKernelGGL((ssd_chunk_scan<N, true, false>), grid, dim3(kThreads), sm.total, st, a, geo);
    else if (hd) hipLaunchKernelGGL((ssd_chunk_scan<N, false, true>), grid, dim3(kThreads), sm.total, st, a, geo);
    else hipLaunchKernelGGL((ssd_chunk_scan<N, false, false>), grid, dim3(kThreads), sm.total, st, a, geo);
    profile_mark(st);
    return hipGetLastError();
}

}  // namespace

const char* ssd_unsupported_reason(int L, int H, int P, int N, int Q, bool bf16) {
    if (!bf16) return "SSD supports bf16 I/O only";
    if (P != kP) return "SSD supports head dim P = 64 only";
    if (N != 64 && N != 128) return "SSD supports N = 64 or 128";
    if (Q < 32 || Q > 256 || Q % 32 != 0) return "SSD chunk must be a multiple of 32 in [32, 256]";
    if (H > 65535) return "H must be <= 65535";
    if (L < 0) return "L must be >= 0";
    return "";
}

size_t ssd_workspace_bytes(int B, int L, int H, int P, int N, int Q) {
    (void)P;
    const SsdGeom g = ssd_geom(B, L, H, Q);
    if (g.K <= 1) return 0;
    return (ws_hagg(B, H, g.K, N) + (size_t)B * H * (g.K - 1)) * sizeof(float);
}

hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t st) {
    switch (a.N) {
        case 64: return launch_n<64>(a, st);
        case 128: return launch_n<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
