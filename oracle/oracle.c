/*
 * fp64 CPU oracle for the selective state-space scan -- plain loops, libm exp.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path. It shares no code
 * with the HIP library.
 *
 * What is computed, and where it comes from:
 *  - The selective SSM recurrence of Gu & Dao, "Mamba: Linear-Time Sequence
 *    Modeling with Selective State Spaces" (2023; listed in the references of
 *    the ssm-bench README): per (batch, channel) a state of N values evolves
 *    with input-dependent step Delta_t and input-dependent B_t, C_t
 *    ("Efficient Sequence Modeling: From S4 to Mamba-3", section 03 System,
 *    mamba_minimal.py: "selectivity", explicit time-loop scan).
 *  - Discretisation by exponential-Euler: Abar = exp(Delta*A), Bbar = Delta*B
 *    (same page, section 04 Approach and section 09 Validation: Mamba-3
 *    reduces to exponential-Euler when lambda = 1, theta = 0).
 *  - Output y = C.h + D*x, then gated by silu(z) = z*sigmoid(z) (the gated
 *    block of Gu & Dao 2023; gate applied after the skip term).
 *  - SSD (Mamba-2): A is one scalar per head and the state per head is an
 *    (N, P) matrix; the chunked form splits L into chunks, computes the
 *    intra-chunk part as decayed-attention matrix products and carries the
 *    (N, P) state from chunk to chunk (same page, section 03, mamba2_minimal.py;
 *    section 04 "Chunked SSD with a sequential reference"; Dao & Gu 2024,
 *    "Transformers are SSMs", listed in the ssm-bench references).
 *  - step(): the same recurrence advanced by one token (section 03,
 *    mamba_minimal.py "incremental step()"; section 09 "step() equals a full
 *    forward").
 */
#include "oracle.h"

#include <complex.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n <= 0) n = omp_get_num_procs();
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^{-z}) */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* y = (C.h + D x) * silu(z), with the optional parts left out when absent. */
static double finish_output(double ch, const double* Dskip, long dix, double xv,
                            const double* z, long zix) {
    double v = ch;
    if (Dskip) v += Dskip[dix] * xv;
    if (z) v *= silu(z[zix]);
    return v;
}

static int bad_dims(int a, int b, int c, int d) { return a < 0 || b < 0 || c < 0 || d < 0; }

/* ---------------------------------------------------------------- O1 ---- */
int oracle_scan(int B, int L, int D, int N,
                const double* x, const double* delta, const double* A,
                const double* Bm, const double* Cm, const double* Dskip,
                const double* z, const double* h0, double* y, double* h_final) {
    if (bad_dims(B, L, D, N)) return -1;
    if ((long)B * L * D > 0 && (!x || !delta || !y)) return -1;
    if ((long)D * N > 0 && !A) return -1;
    if ((long)B * L * N > 0 && (!Bm || !Cm)) return -1;
    long units = (long)B * D;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
        long b = u / D, d = u % D;
        double* h = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));
        for (int n = 0; n < N; ++n) h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
        for (long t = 0; t < L; ++t) {
            long i = (b * L + t) * D + d;        /* [B,L,D] */
            const double* Bt = Bm + (b * L + t) * N; /* [B,L,N] */
            const double* Ct = Cm + (b * L + t) * N;
            double dt = delta[i], xv = x[i];
            double ch = 0.0;
            for (int n = 0; n < N; ++n) {
                double abar = exp(dt * A[d * N + n]); /* exponential-Euler */
                h[n] = abar * h[n] + dt * Bt[n] * xv;
                ch += Ct[n] * h[n];
            }
            y[i] = finish_output(ch, Dskip, d, xv, z, i);
        }
        if (h_final)
            for (int n = 0; n < N; ++n) h_final[(b * D + d) * N + n] = h[n];
        free(h);
    }
    return 0;
}

/* ---------------------------------------------------------------- O2 ---- */
int oracle_ssd_seq(int B, int L, int H, int P, int N,
                   const double* x, const double* delta, const double* A,
                   const double* Bm, const double* Cm, const double* Dskip,
                   const double* z, const double* h0, double* y, double* h_final) {
    if (bad_dims(B, L, H, P) || N < 0) return -1;
    long units = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
        long b = u / H, hh = u % H;
        long NP = (long)N * P;
        double* S = (double*)malloc(sizeof(double) * (NP > 0 ? NP : 1)); /* S[n][p] */
        for (long k = 0; k < NP; ++k) S[k] = h0 ? h0[(b * H + hh) * NP + k] : 0.0;
        for (long t = 0; t < L; ++t) {
            double dt = delta[(b * L + t) * H + hh];
            double abar = exp(dt * A[hh]);
            const double* Bt = Bm + (b * L + t) * N;
            const double* Ct = Cm + (b * L + t) * N;
            const double* xt = x + ((b * L + t) * H + hh) * P;
            for (int n = 0; n < N; ++n)
                for (int p = 0; p < P; ++p)
                    S[n * P + p] = abar * S[n * P + p] + dt * Bt[n] * xt[p];
            for (int p = 0; p < P; ++p) {
                double ch = 0.0;
                for (int n = 0; n < N; ++n) ch += Ct[n] * S[n * P + p];
                long i = ((b * L + t) * H + hh) * P + p;
                y[i] = finish_output(ch, Dskip, hh, xt[p], z, i);
            }
        }
        if (h_final)
            for (long k = 0; k < NP; ++k) h_final[(b * H + hh) * NP + k] = S[k];
        free(S);
    }
    return 0;
}

/* ---------------------------------------------------------------- O3 ----
 * Chunk c covers t in [cQ, min((c+1)Q, L)). With lambda_k = Delta_k*A_h and
 * s_i the inclusive in-chunk prefix sum of lambda:
 *   Y_diag[i] = sum_{j<=i} (C_i . B_j) exp(s_i - s_j) Delta_j x_j
 *   Y_off[i]  = exp(s_i) C_i . S_in
 *   S_out     = exp(s_last) S_in + sum_j exp(s_last - s_j) Delta_j B_j (x) x_j
 * The decay from j to i excludes step j's own factor (it is applied when
 * Delta_j B_j x_j enters the state).
 */
int oracle_ssd_chunked(int B, int L, int H, int P, int N, int Q,
                       const double* x, const double* delta, const double* A,
                       const double* Bm, const double* Cm, const double* Dskip,
                       const double* z, const double* h0, double* y, double* h_final) {
    if (bad_dims(B, L, H, P) || N < 0 || Q < 1) return -1;
    long units = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
        long b = u / H, hh = u % H;
        long NP = (long)N * P;
        double* S = (double*)malloc(sizeof(double) * (NP > 0 ? NP : 1));
        double* Snew = (double*)malloc(sizeof(double) * (NP > 0 ? NP : 1));
        double* s = (double*)malloc(sizeof(double) * Q);
        double* G = (double*)malloc(sizeof(double) * (size_t)Q * Q); /* C_i . B_j */
        for (long k = 0; k < NP; ++k) S[k] = h0 ? h0[(b * H + hh) * NP + k] : 0.0;
        for (long c0 = 0; c0 < L; c0 += Q) {
            int len = (int)((L - c0) < Q ? (L - c0) : Q);
            double acc = 0.0;
            for (int i = 0; i < len; ++i) {
                acc += delta[(b * L + c0 + i) * H + hh] * A[hh];
                s[i] = acc;
            }
            for (int i = 0; i < len; ++i)
                for (int j = 0; j <= i; ++j) {
                    double g = 0.0;
                    for (int n = 0; n < N; ++n)
                        g += Cm[(b * L + c0 + i) * N + n] * Bm[(b * L + c0 + j) * N + n];
                    G[i * Q + j] = g;
                }
            for (int i = 0; i < len; ++i) {
                long ti = b * L + c0 + i;
                for (int p = 0; p < P; ++p) {
                    double yd = 0.0;
                    for (int j = 0; j <= i; ++j) {
                        long tj = b * L + c0 + j;
                        yd += G[i * Q + j] * exp(s[i] - s[j]) * delta[tj * H + hh] *
                              x[(tj * H + hh) * P + p];
                    }
                    double yo = 0.0;
                    for (int n = 0; n < N; ++n) yo += Cm[ti * N + n] * S[n * P + p];
                    yo *= exp(s[i]);
                    long ix = (ti * H + hh) * P + p;
                    y[ix] = finish_output(yd + yo, Dskip, hh, x[ix], z, ix);
                }
            }
            double slast = s[len - 1];
            for (int n = 0; n < N; ++n)
                for (int p = 0; p < P; ++p) {
                    double v = exp(slast) * S[n * P + p];
                    for (int j = 0; j < len; ++j) {
                        long tj = b * L + c0 + j;
                        v += exp(slast - s[j]) * delta[tj * H + hh] * Bm[tj * N + n] *
                             x[(tj * H + hh) * P + p];
                    }
                    Snew[n * P + p] = v;
                }
            memcpy(S, Snew, sizeof(double) * NP);
        }
        if (h_final)
            for (long k = 0; k < NP; ++k) h_final[(b * H + hh) * NP + k] = S[k];
        free(S); free(Snew); free(s); free(G);
    }
    return 0;
}

/* ---------------------------------------------------------------- O4 ---- */
int oracle_step(int B, int D, int N, double* state,
                const double* x, const double* delta, const double* A,
                const double* Bm, const double* Cm, const double* Dskip,
                const double* z, double* y) {
    if (bad_dims(B, D, N, 0)) return -1;
    long units = (long)B * D;
#pragma omp parallel for schedule(static)
    for (long u = 0; u < units; ++u) {
        long b = u / D, d = u % D;
        double dt = delta[u], xv = x[u];
        double* h = state + u * N;
        double ch = 0.0;
        for (int n = 0; n < N; ++n) {
            h[n] = exp(dt * A[d * N + n]) * h[n] + dt * Bm[b * N + n] * xv;
            ch += Cm[b * N + n] * h[n];
        }
        y[u] = finish_output(ch, Dskip, d, xv, z, u);
    }
    return 0;
}

int oracle_ssd_step(int B, int H, int P, int N, double* state,
                    const double* x, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, double* y) {
    if (bad_dims(B, H, P, N)) return -1;
    long units = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long u = 0; u < units; ++u) {
        long b = u / H, hh = u % H;
        double dt = delta[u];
        double abar = exp(dt * A[hh]);
        double* S = state + u * (long)N * P;
        const double* xt = x + u * P;
        for (int n = 0; n < N; ++n)
            for (int p = 0; p < P; ++p)
                S[n * P + p] = abar * S[n * P + p] + dt * Bm[b * N + n] * xt[p];
        for (int p = 0; p < P; ++p) {
            double ch = 0.0;
            for (int n = 0; n < N; ++n) ch += Cm[b * N + n] * S[n * P + p];
            y[u * P + p] = finish_output(ch, Dskip, hh, xt[p], z, u * P + p);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- O5 ----
 * Unrolled state, every product written out:
 *   h_T = (prod_{k=0..T} a_k) h0 + sum_{s<=T} (prod_{k=s+1..T} a_k) Delta_s B_s x_s
 * with a_k = exp(Delta_k A). O(L^2) per state element: tiny shapes only.
 */
int oracle_scan_unroll(int B, int L, int D, int N,
                       const double* x, const double* delta, const double* A,
                       const double* Bm, const double* Cm, const double* Dskip,
                       const double* z, const double* h0, double* y, double* h_final) {
    if (bad_dims(B, L, D, N)) return -1;
    for (long b = 0; b < B; ++b)
        for (long d = 0; d < D; ++d)
            for (long T = 0; T < L; ++T) {
                long iT = (b * L + T) * D + d;
                double ch = 0.0;
                for (int n = 0; n < N; ++n) {
                    double hT = 0.0;
                    if (h0) {
                        double pr = 1.0;
                        for (long k = 0; k <= T; ++k)
                            pr *= exp(delta[(b * L + k) * D + d] * A[d * N + n]);
                        hT += pr * h0[(b * D + d) * N + n];
                    }
                    for (long s2 = 0; s2 <= T; ++s2) {
                        double pr = 1.0;
                        for (long k = s2 + 1; k <= T; ++k)
                            pr *= exp(delta[(b * L + k) * D + d] * A[d * N + n]);
                        long is = (b * L + s2) * D + d;
                        hT += pr * delta[is] * Bm[(b * L + s2) * N + n] * x[is];
                    }
                    ch += Cm[(b * L + T) * N + n] * hT;
                    if (h_final && T == L - 1) h_final[(b * D + d) * N + n] = hT;
                }
                y[iT] = finish_output(ch, Dskip, d, x[iT], z, iT);
            }
    if (L == 0 && h_final)
        for (long k = 0; k < (long)B * D * N; ++k) h_final[k] = h0 ? h0[k] : 0.0;
    return 0;
}

int oracle_ssd_unroll(int B, int L, int H, int P, int N,
                      const double* x, const double* delta, const double* A,
                      const double* Bm, const double* Cm, const double* Dskip,
                      const double* z, const double* h0, double* y, double* h_final) {
    if (bad_dims(B, L, H, P) || N < 0) return -1;
    long NP = (long)N * P;
    for (long b = 0; b < B; ++b)
        for (long hh = 0; hh < H; ++hh)
            for (long T = 0; T < L; ++T)
                for (int p = 0; p < P; ++p) {
                    long iT = ((b * L + T) * H + hh) * P + p;
                    double ch = 0.0;
                    for (int n = 0; n < N; ++n) {
                        double hT = 0.0;
                        if (h0) {
                            double pr = 1.0;
                            for (long k = 0; k <= T; ++k)
                                pr *= exp(delta[(b * L + k) * H + hh] * A[hh]);
                            hT += pr * h0[(b * H + hh) * NP + n * P + p];
                        }
                        for (long s2 = 0; s2 <= T; ++s2) {
                            double pr = 1.0;
                            for (long k = s2 + 1; k <= T; ++k)
                                pr *= exp(delta[(b * L + k) * H + hh] * A[hh]);
                            hT += pr * delta[(b * L + s2) * H + hh] * Bm[(b * L + s2) * N + n] *
                                  x[((b * L + s2) * H + hh) * P + p];
                        }
                        ch += Cm[(b * L + T) * N + n] * hT;
                        if (h_final && T == L - 1) h_final[(b * H + hh) * NP + n * P + p] = hT;
                    }
                    y[iT] = finish_output(ch, Dskip, hh, x[iT], z, iT);
                }
    if (L == 0 && h_final)
        for (long k = 0; k < (long)B * H * NP; ++k) h_final[k] = h0 ? h0[k] : 0.0;
    return 0;
}

/* ------------------------------------------------------------- O6 -------
 * Gradient of O1 for training (the training workloads of "Characterizing the
 * Behavior of Training Mamba-based State Space Models on GPUs", abstract, and
 * the training-step sweep of "Efficient Sequence Modeling: From S4 to
 * Mamba-3", section 05 Evaluation). The pages do not write the backward pass
 * out; it is the chain rule applied to O1, taken here in reverse mode.
 *
 * For the scalar loss l = sum(dy * y) + sum(dh_final * h_final), every output
 * is the partial derivative of l with respect to the matching input. Per
 * (b, d), with a_t[n] = exp(delta_t A[d,n]) and v_t = C_t . h_t + D x_t:
 *   y_t = v_t silu(z_t)                => dv_t = dy_t silu(z_t),
 *                                        dz_t = dy_t v_t silu'(z_t),
 *                                        silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
 *   adjoint of the state, backwards:     g_t = dv_t C_t + a_{t+1} g_{t+1},
 *                                        with a_L g_L taken as dh_final
 *   h_t = a_t h_{t-1} + delta_t B_t x_t => dA[d,n]    += g_t[n] a_t[n] h_{t-1}[n] delta_t
 *                                        ddelta_t    += g_t[n] (A[d,n] a_t[n] h_{t-1}[n] + B_t[n] x_t)
 *                                        dx_t        += g_t[n] delta_t B_t[n]  (+ dv_t D)
 *                                        dB_t[n]     += g_t[n] delta_t x_t     (summed over d)
 *                                        dC_t[n]     += dv_t h_t[n]           (summed over d)
 *                                        dD[d]       += dv_t x_t
 *                                        dh0         =  a_0 g_0
 * dDskip is written only when Dskip is given, dz only when z is given; dh0 may be
 * NULL. dh_final NULL means zero. The states of each (b, d) are kept for the
 * whole sequence (L + 1 rows of N), so this is for test sizes. */
int oracle_scan_bwd(int B, int L, int D, int N,
                    const double* x, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, const double* h0,
                    const double* dy, const double* dh_final,
                    double* dx, double* ddelta, double* dA, double* dBm, double* dCm,
                    double* dDskip, double* dz, double* dh0) {
    if (bad_dims(B, L, D, N)) return -1;
    if ((long)B * L * D > 0 && (!x || !delta || !dy || !dx || !ddelta)) return -1;
    if ((long)D * N > 0 && (!A || !dA)) return -1;
    if ((long)B * L * N > 0 && (!Bm || !Cm || !dBm || !dCm)) return -1;
    if ((Dskip && !dDskip) || (z && !dz)) return -1;
    const long bln = (long)B * L * N;
    const int nthr = oracle_get_threads();
    /* per-thread sums of dB and dC: B and C are shared by every channel */
    double* part = (double*)calloc((size_t)nthr * 2 * (bln > 0 ? bln : 1), sizeof(double));
    if (!part) return -1;
    for (long k = 0; k < (long)D * N; ++k) dA[k] = 0.0;
    if (Dskip)
        for (long d = 0; d < D; ++d) dDskip[d] = 0.0;
#pragma omp parallel num_threads(nthr)
    {
#ifdef _OPENMP
        const int tid = omp_get_thread_num();
#else
        const int tid = 0;
#endif
        double* pB = part + (size_t)tid * 2 * bln;
        double* pC = pB + bln;
        double* hs = (double*)malloc(sizeof(double) * ((size_t)(L + 1) * N + 1)); /* hs[t + 1] = h_t */
        double* c = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));         /* a_{t+1} g_{t+1} */
#pragma omp for schedule(static)
        for (long d = 0; d < D; ++d) {
            for (long b = 0; b < B; ++b) {
                for (int n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
                for (long t = 0; t < L; ++t) {
                    long i = (b * L + t) * D + d;
                    const double* Bt = Bm + (b * L + t) * N;
                    for (int n = 0; n < N; ++n)
                        hs[(t + 1) * N + n] =
                            exp(delta[i] * A[d * N + n]) * hs[t * N + n] + delta[i] * Bt[n] * x[i];
                }
                for (int n = 0; n < N; ++n) c[n] = dh_final ? dh_final[(b * D + d) * N + n] : 0.0;
                for (long t = L - 1; t >= 0; --t) {
                    long i = (b * L + t) * D + d;
                    const double* Bt = Bm + (b * L + t) * N;
                    const double* Ct = Cm + (b * L + t) * N;
                    const double* hprev = hs + t * N;
                    const double* hcur = hs + (t + 1) * N;
                    double dt = delta[i], xv = x[i];
                    double v = 0.0;
                    for (int n = 0; n < N; ++n) v += Ct[n] * hcur[n];
                    if (Dskip) v += Dskip[d] * xv;
                    double dv = dy[i];
                    if (z) {
                        double s = 1.0 / (1.0 + exp(-z[i]));
                        dz[i] = dy[i] * v * s * (1.0 + z[i] * (1.0 - s));
                        dv = dy[i] * z[i] * s;
                    }
                    double gx = 0.0, gdt = 0.0;
                    if (Dskip) {
                        gx = dv * Dskip[d];
                        dDskip[d] += dv * xv;
                    }
                    for (int n = 0; n < N; ++n) {
                        double g = c[n] + dv * Ct[n];
                        double abar = exp(dt * A[d * N + n]);
                        pC[(b * L + t) * N + n] += dv * hcur[n];
                        pB[(b * L + t) * N + n] += g * dt * xv;
                        gx += g * dt * Bt[n];
                        gdt += g * (A[d * N + n] * abar * hprev[n] + Bt[n] * xv);
                        dA[d * N + n] += g * abar * hprev[n] * dt;
                        c[n] = abar * g;
                    }
                    dx[i] = gx;
                    ddelta[i] = gdt;
                }
                if (dh0)
                    for (int n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = c[n];
            }
        }
        free(hs);
        free(c);
    }
    for (long k = 0; k < bln; ++k) {
        double sb = 0.0, sc = 0.0;
        for (int r = 0; r < nthr; ++r) {
            sb += part[(size_t)r * 2 * bln + k];
            sc += part[(size_t)r * 2 * bln + bln + k];
        }
        dBm[k] = sb;
        dCm[k] = sc;
    }
    free(part);
    return 0;
}

/* ------------------------------------------------------------- O7 -------
 * Discretisation variants of O1 and O4.
 *  - Delta preprocessing: Delta = Delta_raw + delta_bias[d] (when given), then
 *    softplus(Delta) = log(1 + e^Delta) when delta_softplus is set (reading: the
 *    usual Mamba input to the scan; the pages draw Delta through a softplus).
 *  - Exact zero-order hold ("Efficient Sequence Modeling: From S4 to Mamba-3",
 *    section 03 (s4_minimal.py), section 04 "Math-verified discretization" and
 *    question Q01): for diagonal A, Abar = exp(z) and Bbar = Delta B (e^z - 1)/z
 *    with z = Delta A, switching to the Taylor series 1 + z/2 + z^2/6 for
 *    |z| < 1e-4 to avoid 0/0, as the page describes. Exponential-Euler keeps
 *    Bbar = Delta B. */
static double softplus(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }

/* (e^z - 1)/z, the page's way */
static double zoh_phi(double z) {
    if (fabs(z) < 1e-4) return 1.0 + z / 2.0 + z * z / 6.0;
    return (exp(z) - 1.0) / z;
}

/* one step's discretisation of channel d, state index n */
static void discretise(int disc, double dt, double a, double* abar, double* bcoef) {
    *abar = exp(dt * a);
    *bcoef = disc == 1 ? dt * zoh_phi(dt * a) : dt;
}

static double pre_delta(double raw, const double* delta_bias, long d, int delta_softplus) {
    double dt = raw;
    if (delta_bias) dt += delta_bias[d];
    if (delta_softplus) dt = softplus(dt);
    return dt;
}

int oracle_scan_disc(int B, int L, int D, int N, int disc, const double* delta_bias, int delta_softplus,
                     const double* x, const double* delta, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     const double* z, const double* h0, double* y, double* h_final) {
    if (bad_dims(B, L, D, N) || (disc != 0 && disc != 1)) return -1;
    if ((long)B * L * D > 0 && (!x || !delta || !y)) return -1;
    if ((long)D * N > 0 && !A) return -1;
    if ((long)B * L * N > 0 && (!Bm || !Cm)) return -1;
    long units = (long)B * D;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
        long b = u / D, d = u % D;
        double* st = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));
        for (int n = 0; n < N; ++n) st[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
        for (long t = 0; t < L; ++t) {
            long i = (b * L + t) * D + d;
            const double* Brow = Bm + (b * L + t) * N;
            const double* Crow = Cm + (b * L + t) * N;
            double dt = pre_delta(delta[i], delta_bias, d, delta_softplus), xv = x[i];
            double ch = 0.0;
            for (int n = 0; n < N; ++n) {
                double abar, bcoef;
                discretise(disc, dt, A[d * N + n], &abar, &bcoef);
                st[n] = abar * st[n] + bcoef * Brow[n] * xv;
                ch += Crow[n] * st[n];
            }
            y[i] = finish_output(ch, Dskip, d, xv, z, i);
        }
        if (h_final)
            for (int n = 0; n < N; ++n) h_final[(b * D + d) * N + n] = st[n];
        free(st);
    }
    return 0;
}

int oracle_step_disc(int B, int D, int N, int disc, const double* delta_bias, int delta_softplus,
                     double* state, const double* x, const double* delta, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     const double* z, double* y) {
    if (bad_dims(B, D, N, 0) || (disc != 0 && disc != 1)) return -1;
    long units = (long)B * D;
#pragma omp parallel for schedule(static)
    for (long u = 0; u < units; ++u) {
        long b = u / D, d = u % D;
        double dt = pre_delta(delta[u], delta_bias, d, delta_softplus), xv = x[u];
        double* h = state + u * N;
        double ch = 0.0;
        for (int n = 0; n < N; ++n) {
            double abar, bcoef;
            discretise(disc, dt, A[d * N + n], &abar, &bcoef);
            h[n] = abar * h[n] + bcoef * Bm[b * N + n] * xv;
            ch += Cm[b * N + n] * h[n];
        }
        y[u] = finish_output(ch, Dskip, d, xv, z, u);
    }
    return 0;
}

/* ------------------------------------------------------------- O8 -------
 * Mamba-3 ("Efficient Sequence Modeling: From S4 to Mamba-3", section 03
 * System, mamba3_minimal.py, and section 04 "Complex transitions for state
 * tracking"): complex diagonal transitions A = Are + i theta (the page writes
 * A = -exp(a) + i theta; Are is passed as the value -exp(a)) with a
 * data-dependent exponential-trapezoidal rule weighted by lam. The pages name
 * the rule and pin its reduction to exponential-Euler at lam = 1, theta = 0
 * but do not write it out; the reading taken is the trapezoidal rule applied to
 * the exact solution over one step,
 *   h(t) = e^{Delta A} h(t-1) + integral_0^Delta e^{A (Delta - s)} B x ds,
 * with the integrand's two endpoint values e^{Delta A} B_{t-1} x_{t-1} and
 * B_t x_t weighted (1 - lam) and lam (lam = 1/2: the trapezoidal rule; lam = 1:
 * exponential-Euler). The output reads the real part of the state. */
int oracle_scan3(int B, int L, int D, int N,
                 const double* x, const double* delta, const double* lam,
                 const double* Are, const double* theta,
                 const double* Bm, const double* Cm, const double* Dskip, const double* z,
                 const double* h0, const double* x_prev, const double* B_prev,
                 double* y, double* h_final) {
    if (bad_dims(B, L, D, N)) return -1;
    if ((long)B * L * D > 0 && (!x || !delta || !lam || !y)) return -1;
    if ((long)D * N > 0 && (!Are || !theta)) return -1;
    if ((long)B * L * N > 0 && (!Bm || !Cm)) return -1;
    if ((x_prev == NULL) != (B_prev == NULL)) return -1;
    long units = (long)B * D;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
        long b = u / D, d = u % D;
        double complex* h = (double complex*)malloc(sizeof(double complex) * (N > 0 ? N : 1));
        for (int n = 0; n < N; ++n) {
            long k = ((b * D + d) * N + n) * 2;
            h[n] = h0 ? h0[k] + I * h0[k + 1] : 0.0;
        }
        double xp = x_prev ? x_prev[b * D + d] : 0.0;   /* x_{t-1} */
        const double* Bp = B_prev ? B_prev + b * N : NULL;  /* B_{t-1} */
        for (long t = 0; t < L; ++t) {
            long i = (b * L + t) * D + d;
            const double* Bt = Bm + (b * L + t) * N;
            const double* Ct = Cm + (b * L + t) * N;
            double dt = delta[i], xv = x[i], lm = lam[i];
            double ch = 0.0;
            for (int n = 0; n < N; ++n) {
                double complex alpha = cexp(dt * (Are[d * N + n] + I * theta[d * N + n]));
                double prev = Bp ? Bp[n] * xp : 0.0;
                h[n] = alpha * h[n] + (1.0 - lm) * dt * alpha * prev + lm * dt * Bt[n] * xv;
                ch += Ct[n] * creal(h[n]);
            }
            y[i] = finish_output(ch, Dskip, d, xv, z, i);
            xp = xv;
            Bp = Bt;
        }
        if (h_final)
            for (int n = 0; n < N; ++n) {
                long k = ((b * D + d) * N + n) * 2;
                h_final[k] = creal(h[n]);
                h_final[k + 1] = cimag(h[n]);
            }
        free(h);
    }
    return 0;
}
