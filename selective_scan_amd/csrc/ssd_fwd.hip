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
// Kernels (one workgroup per (batch, head, super-chunk); a super-chunk is a run
// of consecutive chunks walked in order):
//   ssd_state_agg    (4 waves) every super-chunk but the last: its aggregate
//                    state from a zero start and its total log2 decay;
//   ssd_carry        per (batch, head, state element), a linear walk over the
//                    super-chunks that turns the aggregates into the state
//                    entering each super-chunk (h0 folded in), in place;
//   ssd_chunk_scan   (8 waves) starting from its entering state, for every chunk:
//                    Y_off = diag(e^s) C H, G^T = B C^T, M = G o decay o Delta
//                    (causal), Y_diag = M X, y = (Y_off + Y_diag + D x) silu(z),
//                    then the chunk state S = (w o X)^T B and H <- e^{s_last} H + S.
// The fp32 state H^T (P x N) lives in registers, each wave owning the 16x16 tiles
// it accumulates S into; after every update its bf16 high part and bf16
// remainder are written to LDS, where they are the operands of Y_off.
// Matrix cores: the output phase works on 32-row blocks with
// v_mfma_f32_32x32x16_bf16 (each B / x / state operand fetched from LDS feeds
// twice the flops of a 16x16 tile); the chunk state uses v_mfma_f32_16x16x32_bf16.
// Operands stored in bf16 (B, C, x) enter exactly; operands formed in fp32
// (H, M, w o x) enter as a bf16 high part plus a bf16 remainder, i.e. two MFMAs,
// which keeps about 16 significant bits (one bf16 rounding would cost ~1e-3
// relative error). Where a product contracts over time, its operand is read with
// the LDS transpose read (ds_read_b64_tr_b16), which hands each lane four
// consecutive time steps of one column.
// Below the diagonal, exp2(s_i - s_j) = exp2(s_i - s_r) exp2(s_r - s_j) with r the
// last step of j's 32-step block: one exp per row and a per-column factor staged
// once per chunk (both factors <= 1, so neither can overflow).
// Pipeline per chunk (ssd_chunk_scan): the next chunk's x rows and Delta load
// into registers during the output phase, its B rows during the state phase; the
// wave with the least output work writes the next decay prefix into the second
// of two prefix buffers, and the C rows of a wave's first output block load
// across the barrier; two barriers per chunk.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// LDS-typed pointers keep the address arithmetic in 32 bits
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) u16 lds_u16;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
#ifndef SSM_SSD_TARGET_BLOCKS
#define SSM_SSD_TARGET_BLOCKS 768
#endif
constexpr int kTargetBlocks = SSM_SSD_TARGET_BLOCKS;  // workgroups of the scan kernel
constexpr int kP = 64;              // head dim handled
constexpr int kMaxQ = 256;          // longest chunk
constexpr int kXS = kP + 16;        // LDS row stride (elements) of x rows
constexpr int kPad = 16;            // LDS row padding (elements) of B rows
constexpr int kHPad = 8;            // LDS row padding (elements) of the bf16 state rows
constexpr int kArrays = 5;          // per-step arrays of a prefix buffer: s2, dt, w, cf, es

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v = hi + lo with hi the truncation of v to bf16 (exact) and lo = bf16(v - hi)
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t u = __float_as_uint(v[e]) & 0xffff0000u;
        hi[e] = __builtin_bit_cast(__bf16, (u16)(u >> 16));
        lo[e] = (__bf16)(v[e] - __uint_as_float(u));
    }
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const lds_u16* p) { return *reinterpret_cast<const lds_bf16x8*>(p); }
__device__ __forceinline__ f32x4 ld_f32x4(const lds_f32* p) { return *reinterpret_cast<const lds_f32x4*>(p); }

// Transposed operand read from a row-major [k][m] bf16 array in LDS (row stride
// `rs` elements): lane i of each 16-lane group receives rows k0 .. k0+3 of column
// m0 + i. Each lane of the group points at row k0 + i/4, columns m0 + 4(i%4) ...+3.
__device__ __forceinline__ bf16x4 ld_tr4(const lds_u16* base, int rs, int k0, int m0) {
    const int i = threadIdx.x & 15;
    const lds_u16* p = base + (k0 + (i >> 2)) * rs + m0 + 4 * (i & 3);
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

struct SsdGeom {
    int Q;    // chunk length
    int Qp;   // chunk length rounded up to the 32-row blocks the kernels tile by
    int C;    // chunks per sequence
    int cps;  // chunks per super-chunk
    int K;    // super-chunks per sequence
};

SsdGeom ssd_geom(int B, int L, int H, int Q) {
    SsdGeom g;
    g.Q = Q;
    g.Qp = (Q + 31) / 32 * 32;
    g.C = L > 0 ? (L + Q - 1) / Q : 0;
    const long bh = (long)B * H;
    long K = (kTargetBlocks + bh - 1) / bh;
    K = std::max<long>(1, std::min<long>(K, g.C));
    g.cps = g.C > 0 ? (int)((g.C + K - 1) / K) : 1;
    g.K = g.C > 0 ? (g.C + g.cps - 1) / g.cps : 0;
    return g;
}

// Output work of one chunk: up to two items per wave, an item being a 32-row
// block I and npb 32-column blocks of p starting at pb0 (npb = 0: none).
struct OutPlan {
    int8_t I[kWaves][2];
    int8_t pb0[kWaves][2];
    int8_t npb[kWaves][2];
    int8_t pw;  // the least loaded wave: it loads Delta and computes the decay prefix
};

// Longest-processing-time assignment of the items of R row blocks to the 4 SIMDs
// (waves w and w + 4 share SIMD w % 4) and to their waves. Whole row blocks are
// split into single p-blocks, heaviest first, until there are 8 items; an
// item's cost counts its MFMAs (G and Y_diag per column block, Y_off).
OutPlan out_plan(int R, int N) {
    struct Item { int I, pb0, npb; };
    Item items[2 * kMaxQ / 32];
    int n = 0;
    for (int I = 0; I < R; ++I) items[n++] = {I, 0, 2};
    for (int I = R - 1; I >= 0 && n < kWaves; --I) {
        items[I] = {I, 0, 1};
        items[n++] = {I, 1, 1};
    }
    auto cost = [N](const Item& it) { return (it.I + 1) * (N / 16 + 4 * it.npb) + 2 * (N / 16) * it.npb; };
    std::sort(items, items + n, [&](const Item& x, const Item& y) { return cost(x) > cost(y); });
    OutPlan p{};
    int load_w[kWaves] = {}, used[kWaves] = {}, load_s[4] = {};
    for (int k = 0; k < n; ++k) {
        int best = -1;
        for (int w = 0; w < kWaves; ++w) {
            if (used[w] == 2) continue;
            if (best < 0 || load_s[w % 4] < load_s[best % 4] ||
                (load_s[w % 4] == load_s[best % 4] && load_w[w] < load_w[best]))
                best = w;
        }
        const int c = cost(items[k]);
        p.I[best][used[best]] = (int8_t)items[k].I;
        p.pb0[best][used[best]] = (int8_t)items[k].pb0;
        p.npb[best][used[best]] = (int8_t)items[k].npb;
        ++used[best];
        load_w[best] += c;
        load_s[best % 4] += c;
    }
    p.pw = 0;
    for (int w = 1; w < kWaves; ++w)
        if (load_w[w] < load_w[p.pw]) p.pw = (int8_t)w;
    return p;
}

// LDS layout (bytes), per workgroup
struct Smem {
    int xs, bs, hh, hl, sv, red, tot, total;
};

template <int N>
__host__ __device__ inline Smem smem_layout(int Q) {
    Smem s;
    s.xs = 0;                              // bf16 [Q][kXS]       x rows of the chunk
    s.bs = s.xs + Q * kXS * 2;             // bf16 [Q][N+kPad]    B rows of the chunk
    s.hh = s.bs + Q * (N + kPad) * 2;      // bf16 [P][N+kHPad]   state H^T, high part
    s.hl = s.hh + kP * (N + kHPad) * 2;    // bf16 [P][N+kHPad]   state H^T, remainder
    s.sv = s.hl + kP * (N + kHPad) * 2;    // f32  [2][kArrays][Q] two prefix buffers
    s.red = s.sv + 2 * kArrays * Q * 4;    // f32  [2]  s_last of each prefix buffer
    s.tot = s.red + 16;                    // f64  [kWaves]  per-wave partial sums
    s.total = s.tot + 8 * kWaves;
    return s;
}

// Per-step arrays of prefix buffer sb: 0 s2 (inclusive log2-decay prefix),
// 1 dt (Delta), 2 w = exp2(s_last - s_t) Delta_t, 3 cf = exp2(s_r - s_t) Delta_t with
// r = t | 31, 4 es = exp2(s_t).
__device__ __forceinline__ lds_f32* sv_arr(lds_t* lds, const Smem& sm, int Q, int sb, int which) {
    return reinterpret_cast<lds_f32*>(lds + sm.sv) + (sb * kArrays + which) * Q;
}
__device__ __forceinline__ const lds_f32* sv_arr(const lds_t* lds, const Smem& sm, int Q, int sb, int which) {
    return reinterpret_cast<const lds_f32*>(lds + sm.sv) + (sb * kArrays + which) * Q;
}
__device__ __forceinline__ float s_last(const lds_t* lds, const Smem& sm, int sb) {
    return reinterpret_cast<const lds_f32*>(lds + sm.red)[sb];
}

// workspace (floats): Hagg [B][H][K-1][P][N], Lam [B][H][K-1]
__host__ __device__ inline size_t ws_hagg(int B, int H, int K, int N) { return (size_t)B * H * (K - 1) * kP * N; }

// Buffer views of one batch row's slabs: x, z, y [L][H][P], Delta [L][H], B, C
// [L][N], each sized to its slab, so a time step t >= L reads zeros and a store
// there is dropped (the ragged tail of the last chunk needs no masking).
// Offsets are bytes within the slab.
struct Views {
    __amdgpu_buffer_rsrc_t x, dl, bm, cm, z, y;
    uint32_t xrow;  // bytes per time step of x, z, y: H P 2
    uint32_t xh;    // offset of head h inside a step: h P 2
    uint32_t drow;  // bytes per time step of Delta: H 2
};

template <int N>
__device__ __forceinline__ Views make_views(const SsdArgs& a, int b, int h) {
    Views v;
    const size_t lhp = (size_t)a.L * a.H * kP;
    const u16* x = static_cast<const u16*>(a.x) + (size_t)b * lhp;
    v.x = make_rsrc(x, (uint32_t)(lhp * 2));
    v.z = make_rsrc(a.z ? static_cast<const u16*>(a.z) + (size_t)b * lhp : x, (uint32_t)(lhp * 2));
    v.y = make_rsrc(static_cast<u16*>(a.y) + (size_t)b * lhp, (uint32_t)(lhp * 2));
    v.dl = make_rsrc(static_cast<const u16*>(a.delta) + (size_t)b * a.L * a.H, (uint32_t)((size_t)a.L * a.H * 2));
    v.bm = make_rsrc(static_cast<const u16*>(a.Bm) + (size_t)b * a.L * N, (uint32_t)((size_t)a.L * N * 2));
    v.cm = make_rsrc(static_cast<const u16*>(a.Cm) + (size_t)b * a.L * N, (uint32_t)((size_t)a.L * N * 2));
    v.xrow = (uint32_t)(a.H * kP * 2);
    v.xh = (uint32_t)(h * kP * 2);
    v.drow = (uint32_t)(a.H * 2);
    return v;
}

__device__ __forceinline__ u32x4 ld_buf16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Rows of x and B of one chunk (and, in the prefix wave, its Delta) held in registers
// between the global load and the LDS store, for chunks of at most QM steps.
template <int N, int QM>
struct ChunkRows {
    static constexpr int XQ = QM * (kP / 8) / kThreads;  // 16-byte pieces per thread
    static constexpr int BQ = QM * (N / 8) / kThreads;
    u32x4 xv[XQ];
    u32x4 bv[BQ];
    float dv[4];
};

// x rows (and, in wave pw, Delta) of the chunk starting at step t0; rows of
// pieces that start at or past Q are not loaded.
template <int N, int QM>
__device__ __forceinline__ void load_x_rows(const Views& v, int Q, int t0, ChunkRows<N, QM>& cr, int pw) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int k = 0; k < ChunkRows<N, QM>::XQ; ++k) {
        const int q = tid + k * kThreads;
        const int r = q / (kP / 8), c8 = (q % (kP / 8)) * 8;
        if (k * kThreads / (kP / 8) < Q) cr.xv[k] = ld_buf16(v.x, (uint32_t)(t0 + r) * v.xrow + v.xh + 2 * c8);
    }
    if (wave == pw) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = lane * 4 + k;
            cr.dv[k] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(
                v.dl, (int)((uint32_t)(t0 + t) * v.drow + v.xh / kP), 0, 0));
        }
    }
}

template <int N, int QM>
__device__ __forceinline__ void load_b_rows(const Views& v, int Q, int t0, ChunkRows<N, QM>& cr) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < ChunkRows<N, QM>::BQ; ++k) {
        const int q = tid + k * kThreads;
        const int r = q / (N / 8), c8 = (q % (N / 8)) * 8;
        if (k * kThreads / (N / 8) < Q) cr.bv[k] = ld_buf16(v.bm, (uint32_t)((t0 + r) * N + c8) * 2);
    }
}

// x and B rows of a chunk from registers into LDS (rows >= len hold zeros)
template <int N, int QM>
__device__ __forceinline__ void store_xb(lds_t* lds, const Smem& sm, int Q, const ChunkRows<N, QM>& cr) {
    const int tid = threadIdx.x;
    lds_u16* xs = reinterpret_cast<lds_u16*>(lds + sm.xs);
    lds_u16* bs = reinterpret_cast<lds_u16*>(lds + sm.bs);
#pragma unroll
    for (int k = 0; k < ChunkRows<N, QM>::XQ; ++k) {
        const int q = tid + k * kThreads;
        const int r = q / (kP / 8), c8 = (q % (kP / 8)) * 8;
        if (k * kThreads / (kP / 8) < Q && r < Q) *reinterpret_cast<lds_u32x4*>(xs + r * kXS + c8) = cr.xv[k];
    }
#pragma unroll
    for (int k = 0; k < ChunkRows<N, QM>::BQ; ++k) {
        const int q = tid + k * kThreads;
        const int r = q / (N / 8), c8 = (q % (N / 8)) * 8;
        if (k * kThreads / (N / 8) < Q && r < Q) *reinterpret_cast<lds_u32x4*>(bs + r * (N + kPad) + c8) = cr.bv[k];
    }
}

// One wave: the chunk's decay prefix and per-step factors into prefix buffer sb.
// Lane l owns steps 4l .. 4l+3 (Q <= 256); fp64 running sums, then a wave scan.
__device__ __forceinline__ void chunk_prefix(lds_t* lds, const Smem& sm, int Q, int sb, int len, float A2,
                                             const float (&dv)[4]) {
    const int lane = threadIdx.x & 63;
    lds_f32* s2 = sv_arr(lds, sm, Q, sb, 0);
    lds_f32* dt = sv_arr(lds, sm, Q, sb, 1);
    lds_f32* w = sv_arr(lds, sm, Q, sb, 2);
    lds_f32* cf = sv_arr(lds, sm, Q, sb, 3);
    lds_f32* es = sv_arr(lds, sm, Q, sb, 4);
    double loc[4], run = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        run += (double)(dv[k] * A2);
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
            dt[t] = dv[k];
            w[t] = t < len ? exp2_fast(sl - s) * dv[k] : 0.0f;
            cf[t] = t < len ? exp2_fast(r - s) * dv[k] : 0.0f;
            es[t] = exp2_fast(s);
        }
    }
    if (lane == 0) reinterpret_cast<lds_f32*>(lds + sm.red)[sb] = sl;
}

// Chunk state S^T = (w o X)^T B on this wave's tiles: p-block pb = wave % 4 and
// n-blocks nb0 .. nb0 + NBW - 1. Lane holds S^T[p = pb*16 + 4g + r][n = nb*16 + l%16].
template <int N>
struct StateTiles {
    static constexpr int NBW = N / 32;  // n-blocks per wave (8 waves = 4 p-blocks x 2 halves)
    f32x4 acc[NBW];
};

template <int N>
__device__ __forceinline__ void chunk_state(const lds_t* lds, const Smem& sm, int Q, int sb, int len,
                                            StateTiles<N>& st, bool accumulate = false) {
    constexpr int NBW = StateTiles<N>::NBW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int pb = wave & 3, nb0 = (wave >> 2) * NBW;
    const lds_u16* xs = reinterpret_cast<const lds_u16*>(lds + sm.xs);
    const lds_u16* bs = reinterpret_cast<const lds_u16*>(lds + sm.bs);
    const lds_f32* w = sv_arr(lds, sm, Q, sb, 2);
#pragma unroll
    for (int k = 0; k < NBW; ++k)
        if (!accumulate) st.acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    // operands of one 32-step block: x (4 + 4 steps of column p), the weights,
    // and the B operands of this wave's n-blocks
    struct Ops {
        bf16x8 x;
        f32x4 w0, w1;
        bf16x8 b[NBW];
    };
    auto fetch = [&](int kb, Ops& o) {
        const int t = kb * 32 + 8 * g;
        o.x = cat(ld_tr4(xs, kXS, t, pb * 16), ld_tr4(xs, kXS, t + 4, pb * 16));
        o.w0 = ld_f32x4(w + t);
        o.w1 = ld_f32x4(w + t + 4);
#pragma unroll
        for (int k = 0; k < NBW; ++k) {
            const int n0 = (nb0 + k) * 16;
            o.b[k] = cat(ld_tr4(bs, N + kPad, t, n0), ld_tr4(bs, N + kPad, t + 4, n0));
        }
    };
    auto use = [&](const Ops& o) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = (float)o.x[e] * o.w0[e];
            v[e + 4] = (float)o.x[e + 4] * o.w1[e];
        }
        bf16x8 ahi, alo;
        split8(v, ahi, alo);
        // high parts first, then remainders: no two back-to-back MFMAs share an accumulator
#pragma unroll
        for (int k = 0; k < NBW; ++k) st.acc[k] = mfma16(ahi, o.b[k], st.acc[k]);
#pragma unroll
        for (int k = 0; k < NBW; ++k) st.acc[k] = mfma16(alo, o.b[k], st.acc[k]);
    };
    // two operand sets in flight: block kb + 1 is read while block kb is used
    const int kbn = (len + 31) >> 5;
    Ops o0, o1;
    fetch(0, o0);
    for (int kb = 0; kb < kbn; kb += 2) {
        if (kb + 1 < kbn) fetch(kb + 1, o1);
        use(o0);
        if (kb + 1 < kbn) {
            if (kb + 2 < kbn) fetch(kb + 2, o0);
            use(o1);
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
__device__ __forceinline__ void state_update(const lds_t* lds, const Smem& sm, int sb, State<N>& hs,
                                             const StateTiles<N>& st) {
    const float decay = exp2_fast(s_last(lds, sm, sb));
#pragma unroll
    for (int k = 0; k < StateTiles<N>::NBW; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) hs.h[k][r] = __builtin_fmaf(decay, hs.h[k][r], st.acc[k][r]);
}

// bf16 high part and remainder of this wave's state tiles into LDS
template <int N>
__device__ __forceinline__ void state_to_lds(lds_t* lds, const Smem& sm, const State<N>& hs) {
    constexpr int NBW = StateTiles<N>::NBW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int pb = wave & 3, nb0 = (wave >> 2) * NBW;
    lds_u16* hh = reinterpret_cast<lds_u16*>(lds + sm.hh);
    lds_u16* hl = reinterpret_cast<lds_u16*>(lds + sm.hl);
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

// Block coordinates of a 1-D grid of B * K' * H workgroups, heads fastest.
// Workgroups go round-robin to the 8 XCDs (each with its own L2); when the
// count allows, consecutive coordinates are given to one XCD so that all heads
// of a (batch, super-chunk), which read the same B and C rows, share its L2.
__device__ __forceinline__ void block_coords(int H, int Kp, int& h, int& k, int& b) {
    const int total = (int)gridDim.x, id = (int)blockIdx.x;
    const int idp = (total % 8 == 0) ? (id % 8) * (total / 8) + id / 8 : id;
    h = idp % H;
    const int r = idp / H;
    k = r % Kp;
    b = r / Kp;
}

// Aggregate of one super-chunk (all but the last of each (batch, head)), from a
// zero state: S = sum over its steps t of exp2(Lam - s_t) Delta_t B_t (x) x_t,
// with s_t the inclusive log2-decay prefix from the super-chunk's start and Lam
// its total (also written out). The super-chunk is walked in blocks of kAggT
// steps; per block j with total log2 decay S_j the aggregate is rescaled and
// extended, S <- exp2(S_j) S + sum_{t in j} exp2(S_j - s_t) Delta_t B_t (x) x_t,
// with s_t now the prefix inside the block (fp64, rounded once), which is the
// same sum regrouped.
//
// One workgroup of 4 waves per (batch, head, super-chunk). Wave w owns the n
// columns [w N/4, (w+1) N/4) of S^T (P x N) for all 64 p, as 16x16 tiles. Its
// operands per 32-step sub-block: x^T read with the LDS transpose read (exact
// bf16), and (w o B) formed in registers from the transposed B rows and split
// into a bf16 high part and remainder (two MFMAs). Every wave computes the
// block's decay prefix itself (one Delta per lane, an fp64 scan across the
// wave) and keeps its weights in a private LDS slot. Rows of x and B (and the
// Delta of each lane) arrive two blocks ahead of their use in registers.
constexpr int kAggWaves = 4;
constexpr int kAggThreads = 64 * kAggWaves;
constexpr int kAggT = 64;  // steps per staged block

template <int N>
struct AggLds {
    static constexpr int BS = N + kPad;                      // B row stride (elements)
    static constexpr int XS_OFF = 0;                         // bf16 [kAggT][kXS]
    static constexpr int BS_OFF = XS_OFF + kAggT * kXS * 2;  // bf16 [kAggT][BS]
    static constexpr int W_OFF = BS_OFF + kAggT * BS * 2;    // f32 [kAggWaves][kAggT]
    static constexpr int TOTAL = W_OFF + kAggWaves * kAggT * 4;
};

template <int N>
struct AggRows {
    static constexpr int XQ = kAggT * (kP / 8) / kAggThreads;  // 16-byte pieces per thread
    static constexpr int BQ = kAggT * (N / 8) / kAggThreads;
    u32x4 xv[XQ];
    u32x4 bv[BQ];
    uint32_t dl;  // Delta of step `lane` of the block (bf16 bits)
};

template <int N>
__device__ __forceinline__ void agg_load(const Views& v, int t0, AggRows<N>& r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < AggRows<N>::XQ; ++k) {
        const int q = tid + k * kAggThreads;
        const int row = q / (kP / 8), c8 = (q % (kP / 8)) * 8;
        r.xv[k] = ld_buf16(v.x, (uint32_t)(t0 + row) * v.xrow + v.xh + 2 * c8);
    }
#pragma unroll
    for (int k = 0; k < AggRows<N>::BQ; ++k) {
        const int q = tid + k * kAggThreads;
        const int row = q / (N / 8), c8 = (q % (N / 8)) * 8;
        r.bv[k] = ld_buf16(v.bm, (uint32_t)((t0 + row) * N + c8) * 2);
    }
    r.dl = __builtin_amdgcn_raw_buffer_load_b16(v.dl, (int)((uint32_t)(t0 + (tid & 63)) * v.drow + v.xh / kP), 0,
                                                0);
}

// Rows of a block into LDS (rows at or past len as zeros), and this wave's
// weights exp2(S_j - s_t) Delta_t into its slot; returns the block's total log2
// decay S_j (fp64, the same value in every lane).
template <int N>
__device__ __forceinline__ double agg_stage(lds_t* lds, const AggRows<N>& r, int len, float A2) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    lds_u16* xs = reinterpret_cast<lds_u16*>(lds + AggLds<N>::XS_OFF);
    lds_u16* bs = reinterpret_cast<lds_u16*>(lds + AggLds<N>::BS_OFF);
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < AggRows<N>::XQ; ++k) {
        const int q = tid + k * kAggThreads;
        const int row = q / (kP / 8), c8 = (q % (kP / 8)) * 8;
        *reinterpret_cast<lds_u32x4*>(xs + row * kXS + c8) = row < len ? r.xv[k] : zero;
    }
#pragma unroll
    for (int k = 0; k < AggRows<N>::BQ; ++k) {
        const int q = tid + k * kAggThreads;
        const int row = q / (N / 8), c8 = (q % (N / 8)) * 8;
        *reinterpret_cast<lds_u32x4*>(bs + row * AggLds<N>::BS + c8) = row < len ? r.bv[k] : zero;
    }
    const float d = lane < len ? bf16_to_f32((uint16_t)r.dl) : 0.0f;
    double incl = (double)(d * A2);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    const double tot = __shfl(incl, 63, 64);
    lds_f32* w = reinterpret_cast<lds_f32*>(lds + AggLds<N>::W_OFF) + wave * kAggT;
    w[lane] = exp2_fast((float)(tot - incl)) * d;
    return tot;
}

// Three waves per SIMD (at most 168 registers a lane; the compiler would
// otherwise take ~220 with the accumulators in AGPRs and fit two): every
// aggregate of a 768-block launch is resident at once.
template <int N>
__global__ void __launch_bounds__(kAggThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
ssd_state_agg(SsdArgs a, SsdGeom geo) {
    constexpr int NBW = N / 64;  // 16-column n-blocks per wave
    constexpr int BS = AggLds<N>::BS;
    __shared__ __attribute__((aligned(16))) char lds_raw[AggLds<N>::TOTAL];
    lds_t* lds = (lds_t*)lds_raw;
    int h, k, b;
    block_coords(a.H, geo.K - 1, h, k, b);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    const float A2 = a.A[h] * kLog2e;
    const int T0 = k * geo.cps * geo.Q, T1 = min(a.L, (k + 1) * geo.cps * geo.Q);
    const int nblk = (T1 - T0 + kAggT - 1) / kAggT;
    const Views v = make_views<N>(a, b, h);
    const lds_u16* xs = reinterpret_cast<const lds_u16*>(lds + AggLds<N>::XS_OFF);
    const lds_u16* bs = reinterpret_cast<const lds_u16*>(lds + AggLds<N>::BS_OFF);
    const lds_f32* wv = reinterpret_cast<const lds_f32*>(lds + AggLds<N>::W_OFF) + wave * kAggT;
    const int n0w = wave * (N / 4);

    f32x4 acc[4][NBW];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[pb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one block's contraction from LDS, after scaling the aggregate by its decay
    auto contract = [&](float dec) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[pb][nb][r] *= dec;
#pragma unroll
        for (int kb = 0; kb < kAggT / 32; ++kb) {
            const int t = kb * 32 + 8 * g;
            const f32x4 w0 = ld_f32x4(wv + t), w1 = ld_f32x4(wv + t + 4);
            bf16x8 bhi[NBW], blo[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int n0 = n0w + nb * 16;
                const bf16x8 bb = cat(ld_tr4(bs, BS, t, n0), ld_tr4(bs, BS, t + 4, n0));
                float vv[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vv[e] = (float)bb[e] * w0[e];
                    vv[e + 4] = (float)bb[e + 4] * w1[e];
                }
                split8(vv, bhi[nb], blo[nb]);
            }
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const bf16x8 xo = cat(ld_tr4(xs, kXS, t, pb * 16), ld_tr4(xs, kXS, t + 4, pb * 16));
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) acc[pb][nb] = mfma16(xo, bhi[nb], acc[pb][nb]);
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) acc[pb][nb] = mfma16(xo, blo[nb], acc[pb][nb]);
            }
        }
    };

    double lam = 0.0;
    float dec = 1.0f;
    // Two register sets swap roles every block (the body is written out twice so
    // that no in-flight register is copied): while block j is contracted, `nxt`
    // holds the loads of block j + 1 and `nxt2` receives those of block j + 2.
    AggRows<N> ra, rb;
    agg_load<N>(v, T0, rb);
    if (nblk > 1) agg_load<N>(v, T0 + kAggT, ra);
    {
        const double s = agg_stage<N>(lds, rb, min(kAggT, T1 - T0), A2);
        lam += s;
        dec = exp2_fast((float)s);
    }
    auto step = [&](int j, AggRows<N>& nxt, AggRows<N>& nxt2) {
        const int t0 = T0 + j * kAggT;
        __syncthreads();  // rows of block j visible
        if (j + 2 < nblk) agg_load<N>(v, t0 + 2 * kAggT, nxt2);
        contract(dec);
        __syncthreads();  // every read of block j's rows done
        if (j + 1 < nblk) {
            const double s = agg_stage<N>(lds, nxt, min(kAggT, T1 - t0 - kAggT), A2);
            lam += s;
            dec = exp2_fast((float)s);
        }
    };
    for (int j = 0; j < nblk; j += 2) {
        step(j, ra, rb);
        if (j + 1 < nblk) step(j + 1, rb, ra);
    }
    float* out = static_cast<float*>(a.ws) + (((size_t)b * a.H + h) * (geo.K - 1) + k) * kP * N;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[(pb * 16 + 4 * g + r) * N + n0w + nb * 16 + i] = acc[pb][nb][r];
    if (tid == 0) {
        float* lamp = static_cast<float*>(a.ws) + ws_hagg(a.B, a.H, geo.K, N);
        lamp[((size_t)b * a.H + h) * (geo.K - 1) + k] = (float)lam;
    }
}

// Aggregates -> entering states: slot k (k = 0 .. K-2) of (b, h) becomes the
// state entering super-chunk k + 1, H_in(k+1) = exp2(Lam_k) H_in(k) + Hagg_k,
// with H_in(0) = h0 (or zero). One thread per state element (p, n).
template <int N>
__global__ void __launch_bounds__(256)
ssd_carry(const float* __restrict__ h0, float* __restrict__ ws, int B, int H, int K) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    if (e >= kP * N) return;
    const int p = e / N, n = e % N;
    const size_t bh = (size_t)b * H + h;
    float v = h0 ? h0[(bh * N + n) * kP + p] : 0.0f;
    const float* lam = ws + ws_hagg(B, H, K, N) + bh * (K - 1);
    float* slot = ws + bh * (K - 1) * kP * N + e;
    // eight slots loaded before any is written (a load issued after a store would
    // also wait for the store: one memory round trip per 8 super-chunks, not per one)
    for (int k0 = 0; k0 < K - 1; k0 += 8) {
        float sl[8], lm[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = min(k0 + j, K - 2);
            sl[j] = slot[(size_t)k * kP * N];
            lm[j] = lam[k];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (k0 + j < K - 1) {
                v = __builtin_fmaf(exp2_fast(lm[j]), v, sl[j]);
                slot[(size_t)(k0 + j) * kP * N] = v;
            }
        }
    }
}

// C rows of a 32-row block as MFMA operands: lane holds row 32 I + l % 32,
// columns 16 ks + 8 (l / 32) .. +7 for ks = 0 .. N/16 - 1 (zeros past len).
template <int N>
__device__ __forceinline__ void load_c(const Views& v, int t0, int I, bf16x8 (&cop)[N / 16]) {
    const int lane = threadIdx.x & 63;
    const uint32_t off = (uint32_t)((t0 + 32 * I + (lane & 31)) * N + 8 * (lane >> 5)) * 2;
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) cop[ks] = __builtin_bit_cast(bf16x8, ld_buf16(v.cm, off + 32 * ks));
}

// Outputs of one 32-row block I of a chunk for NPB 32-column blocks of p from pb0.
// Lane l: hf = l / 32, c = l % 32. MFMA 32x32x16 layouts: A operand A[c][8 hf + e],
// B operand B[8 hf + e][c], accumulator element r at row 8(r/4) + 4 hf + r%4, column c.
template <int N, int NPB, bool HAS_Z, bool HAS_D, bool PAD>
__device__ __forceinline__ void out_item(const Views& v, const lds_t* lds, const Smem& sm, int Q, int sb,
                                         int t0, int len, int I, int pb0, const bf16x8 (&cop)[N / 16], float Dh) {
    const int lane = threadIdx.x & 63;
    const int hf = lane >> 5, c = lane & 31, gh = (lane >> 4) & 1;
    const lds_u16* xs = reinterpret_cast<const lds_u16*>(lds + sm.xs);
    const lds_u16* bs = reinterpret_cast<const lds_u16*>(lds + sm.bs);
    const lds_u16* hh = reinterpret_cast<const lds_u16*>(lds + sm.hh);
    const lds_u16* hl = reinterpret_cast<const lds_u16*>(lds + sm.hl);
    const lds_f32* s2 = sv_arr(lds, sm, Q, sb, 0);
    const lds_f32* dt = sv_arr(lds, sm, Q, sb, 1);
    const lds_f32* cf = sv_arr(lds, sm, Q, sb, 3);
    const lds_f32* es = sv_arr(lds, sm, Q, sb, 4);
    f32x16 acc[NPB];
#pragma unroll
    for (int q = 0; q < NPB; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;
    // Y_off = C H: rows of H^T (high part and remainder) are the B operands
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks)
#pragma unroll
        for (int q = 0; q < NPB; ++q) {
            const int off = (32 * (pb0 + q) + c) * (N + kHPad) + 16 * ks + 8 * hf;
            acc[q] = mfma32(cop[ks], ld_bf16x8(hh + off), acc[q]);
            acc[q] = mfma32(cop[ks], ld_bf16x8(hl + off), acc[q]);
        }
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
        const f32x4 e4 = ld_f32x4(es + 32 * I + 8 * rq + 4 * hf);
#pragma unroll
        for (int q = 0; q < NPB; ++q)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[q][4 * rq + rr] *= e4[rr];
    }
    // Y_diag = M X over 32-wide column blocks J <= I
    const int i = 32 * I + c;  // this lane's row of G and M
    const float s2i = s2[i];
    for (int J = 0; J <= I && 32 * J < len; ++J) {
        f32x16 g;
#pragma unroll
        for (int r = 0; r < 16; ++r) g[r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < N / 16; ++ks)
            g = mfma32(ld_bf16x8(bs + (32 * J + c) * (N + kPad) + 16 * ks + 8 * hf), cop[ks], g);
        // lane holds G[i][j] for j = 32 J + 8 (r/4) + 4 hf + r % 4
        float m[16];
        if (J < I) {
            const float rowf = exp2_fast(s2i - s2[32 * J + 31]);
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const f32x4 c4 = ld_f32x4(cf + 32 * J + 8 * rq + 4 * hf);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) m[4 * rq + rr] = g[4 * rq + rr] * rowf * c4[rr];
            }
        } else {
            // causal mask j <= i, i.e. 8 (r/4) + r % 4 <= c - 4 hf; columns j >= len
            // only meet rows i >= len, which are never stored (their x rows are zero)
            const int cl = c - 4 * hf;
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int j0 = 32 * J + 8 * rq + 4 * hf;
                const f32x4 sj = ld_f32x4(s2 + j0);
                const f32x4 dj = ld_f32x4(dt + j0);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    m[4 * rq + rr] = (8 * rq + rr <= cl) ? g[4 * rq + rr] * exp2_fast(s2i - sj[rr]) * dj[rr] : 0.0f;
            }
        }
        // two 16-step halves of the block; rows of x in the same (hf, e) -> j order
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
            bf16x8 mhi, mlo;
            split8(m + 8 * ks2, mhi, mlo);
            const int k0 = 32 * J + 16 * ks2 + 4 * hf;
#pragma unroll
            for (int q = 0; q < NPB; ++q) {
                const int m0 = 32 * (pb0 + q) + 16 * gh;
                const bf16x8 xop = cat(ld_tr4(xs, kXS, k0, m0), ld_tr4(xs, kXS, k0 + 8, m0));
                acc[q] = mfma32(mhi, xop, acc[q]);
                acc[q] = mfma32(mlo, xop, acc[q]);
            }
        }
    }
    // epilogue: rows 32 I + 8 (r/4) + 4 hf + r % 4, columns p = 32 (pb0 + q) + c;
    // rows past the sequence end fall outside the y view and are dropped; PAD (a
    // chunk that is not a whole number of blocks): rows at or past the chunk's
    // length, the next chunk's, are not stored
    const uint32_t off0 = (uint32_t)(t0 + 32 * I + 4 * hf) * v.xrow + v.xh + 2 * (32 * pb0 + c);
    // the gate's z values are all loaded before the first y store (a load issued
    // after a store would also wait for that store)
    uint16_t zr[NPB][16];
    if constexpr (HAS_Z) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int q = 0; q < NPB; ++q)
                zr[q][r] = __builtin_amdgcn_raw_buffer_load_b16(
                    v.z, (int)(off0 + (uint32_t)(8 * (r >> 2) + (r & 3)) * v.xrow + 64 * q), 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 32 * I + 8 * (r >> 2) + 4 * hf + (r & 3);
        const uint32_t off = off0 + (uint32_t)(8 * (r >> 2) + (r & 3)) * v.xrow;
#pragma unroll
        for (int q = 0; q < NPB; ++q) {
            float val = acc[q][r];
            if constexpr (HAS_D) val = __builtin_fmaf(Dh, bf16_to_f32(xs[row * kXS + 32 * (pb0 + q) + c]), val);
            if constexpr (HAS_Z) val *= silu(bf16_to_f32(zr[q][r]));
            if (!PAD || row < len)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(val), v.y, (int)(off + 64 * q), 0, 0);
        }
    }
    (void)len;
}

template <int N, bool HAS_Z, bool HAS_D, bool PAD>
__device__ __forceinline__ void run_item(const Views& v, const lds_t* lds, const Smem& sm, int Q, int sb, int t0,
                                         int len, int I, int pb0, int npb, const bf16x8 (&cop)[N / 16], float Dh) {
    if (npb == 2) out_item<N, 2, HAS_Z, HAS_D, PAD>(v, lds, sm, Q, sb, t0, len, I, pb0, cop, Dh);
    else out_item<N, 1, HAS_Z, HAS_D, PAD>(v, lds, sm, Q, sb, t0, len, I, pb0, cop, Dh);
}

// QM: the longest chunk the launch may have (64 or kMaxQ): it sizes the registers that
// carry the next chunk's x and B rows. With QM = 64 they are few enough to be loaded
// before the output phase, which then hides their latency. PAD: the chunk length is
// not a multiple of 32 (its tiles then span the next multiple).
template <int N, bool HAS_Z, bool HAS_D, int QM, bool PAD>
__global__ void __launch_bounds__(kThreads)
ssd_chunk_scan(SsdArgs a, SsdGeom geo, OutPlan plan) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    lds_t* lds = (lds_t*)lds_raw;
    // tiles, LDS rows and prefix arrays span Qp rows; chunks start every Q steps.
    // Rows of a chunk at or past its length (the next chunk's, or past the
    // sequence) enter with zero weight and their outputs are not stored.
    const int Q = geo.Q, Qp = PAD ? geo.Qp : geo.Q;
    const Smem sm = smem_layout<N>(Qp);
    int h, k, b;
    block_coords(a.H, geo.K, h, k, b);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float A2 = a.A[h] * kLog2e;
    const float Dh = HAS_D ? a.Dskip[h] : 0.0f;
    const int c0 = k * geo.cps, c1 = min(geo.C, c0 + geo.cps);
    const int I0 = plan.I[wave][0], P0 = plan.pb0[wave][0], N0 = plan.npb[wave][0];
    const int I1 = plan.I[wave][1], P1 = plan.pb0[wave][1], N1 = plan.npb[wave][1];
    const int PW = plan.pw;

    // state entering this super-chunk: h0 (or zero) for the first, else the
    // slot the carry kernel filled
    State<N> hs;
    {
        const size_t bh = (size_t)b * a.H + h;
        const float* slot = static_cast<const float*>(a.ws) + (bh * (geo.K - 1) + (k - 1)) * kP * N;
#pragma unroll
        for (int kk = 0; kk < StateTiles<N>::NBW; ++kk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int p, n;
                tile_pn<N>(kk, r, p, n);
                float v = 0.0f;
                if (k > 0) v = slot[p * N + n];
                else if (a.h0) v = a.h0[(bh * N + n) * kP + p];
                hs.h[kk][r] = v;
            }
    }
    const Views v = make_views<N>(a, b, h);
    ChunkRows<N, QM> cr;
    bf16x8 cop[N / 16];
    {
        const int len0 = min(Q, a.L - c0 * Q);
        load_x_rows<N, QM>(v, Qp, c0 * Q, cr, PW);
        load_b_rows<N, QM>(v, Qp, c0 * Q, cr);
        if (N0 > 0) load_c<N>(v, c0 * Q, I0, cop);
        state_to_lds<N>(lds, sm, hs);
        if (wave == PW) chunk_prefix(lds, sm, Qp, 0, len0, A2, cr.dv);
        store_xb<N, QM>(lds, sm, Qp, cr);
    }
    const bool last_super = (k == geo.K - 1);
    for (int cc = c0; cc < c1; ++cc) {
        const int sb = (cc - c0) & 1;
        const int t0 = cc * Q;
        const int len = min(Q, a.L - t0);
        const int ln = cc + 1 < c1 ? min(Q, a.L - t0 - Q) : 0;
        __syncthreads();  // rows, prefix and state copy of this chunk visible
        if (ln > 0) {
            load_x_rows<N, QM>(v, Qp, t0 + Q, cr, PW);
            if constexpr (QM <= 64) load_b_rows<N, QM>(v, Qp, t0 + Q, cr);
        }
        if (N0 > 0 && 32 * I0 < len) run_item<N, HAS_Z, HAS_D, PAD>(v, lds, sm, Qp, sb, t0, len, I0, P0, N0, cop, Dh);
        if (N1 > 0 && 32 * I1 < len) {
            load_c<N>(v, t0, I1, cop);
            run_item<N, HAS_Z, HAS_D, PAD>(v, lds, sm, Qp, sb, t0, len, I1, P1, N1, cop, Dh);
        }
        if constexpr (QM > 64) {
            if (ln > 0) load_b_rows<N, QM>(v, Qp, t0 + Q, cr);
        }
        // state after the chunk (not needed after the last chunk of a super-chunk,
        // except at the very end of the sequence for h_final)
        const bool need_state = (cc < c1 - 1) || (last_super && a.h_final != nullptr);
        if (need_state) {
            StateTiles<N> st;
            chunk_state<N>(lds, sm, Qp, sb, len, st);
            state_update<N>(lds, sm, sb, hs, st);
        }
        if (ln > 0) {
            if (wave == PW) chunk_prefix(lds, sm, Qp, sb ^ 1, ln, A2, cr.dv);
            if (N0 > 0) load_c<N>(v, t0 + Q, I0, cop);
        }
        __syncthreads();  // every read of this chunk's rows and state copy done
        if (ln > 0) {
            state_to_lds<N>(lds, sm, hs);
            store_xb<N, QM>(lds, sm, Qp, cr);
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

template <int N, int QM, bool PAD>
void launch_scan(const SsdArgs& a, const SsdGeom& geo, const OutPlan& plan, const Smem& sm, dim3 grid, bool hz,
                 bool hd, hipStream_t st) {
    if (hz && hd) launch((ssd_chunk_scan<N, true, true, QM, PAD>), grid, dim3(kThreads), sm.total, st, a, geo, plan);
    else if (hz) launch((ssd_chunk_scan<N, true, false, QM, PAD>), grid, dim3(kThreads), sm.total, st, a, geo, plan);
    else if (hd) launch((ssd_chunk_scan<N, false, true, QM, PAD>), grid, dim3(kThreads), sm.total, st, a, geo, plan);
    else launch((ssd_chunk_scan<N, false, false, QM, PAD>), grid, dim3(kThreads), sm.total, st, a, geo, plan);
}

template <int N>
hipError_t launch_n(const SsdArgs& a, hipStream_t st) {
    if (a.L == 0) {
        if (a.h_final) {
            const size_t n = (size_t)a.B * a.H * N * a.P;
            launch(copy_state_ssd, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                               a.h0, a.h_final, n);
        }
        return hipGetLastError();
    }
    const SsdGeom geo = ssd_geom(a.B, a.L, a.H, a.Q);
    const Smem sm = smem_layout<N>(geo.Qp);
    const OutPlan plan = out_plan(geo.Qp / 32, N);
    if (geo.K > 1) {
        launch((ssd_state_agg<N>), dim3((unsigned)((geo.K - 1) * a.H * a.B)), dim3(kAggThreads), 0, st, a,
               geo);
        launch((ssd_carry<N>), dim3((kP * N + 255) / 256, a.H, a.B), dim3(256), 0, st,
                           a.h0, static_cast<float*>(a.ws), a.B, a.H, geo.K);
    }
    const bool hz = a.z != nullptr, hd = a.Dskip != nullptr;
    const dim3 grid((unsigned)(geo.K * a.H * a.B));
    const bool pad = geo.Qp != geo.Q;
    if (geo.Qp <= 64) {
        if (pad) launch_scan<N, 64, true>(a, geo, plan, sm, grid, hz, hd, st);
        else launch_scan<N, 64, false>(a, geo, plan, sm, grid, hz, hd, st);
    } else {
        if (pad) launch_scan<N, kMaxQ, true>(a, geo, plan, sm, grid, hz, hd, st);
        else launch_scan<N, kMaxQ, false>(a, geo, plan, sm, grid, hz, hd, st);
    }
    return hipGetLastError();
}

}  // namespace

const char* ssd_unsupported_reason(int L, int H, int P, int N, int Q, bool bf16) {
    if (!bf16) return "SSD supports bf16 I/O only";
    if (P != kP) return "SSD supports head dim P = 64 only";
    if (N != 64 && N != 128) return "SSD supports N = 64 or 128";
    if (Q < 1 || Q > kMaxQ) return "SSD chunk must be in [1, 256]";
    if (H > 65535) return "H must be <= 65535";
    if (L < 0) return "L must be >= 0";
    if ((long long)L * H * P * 2 > 0x7fffffffLL) return "L * H * P * 2 must be < 2^31 (bytes of one batch row of x)";
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
