/*
 * fp64 CPU oracle for the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this: only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header, table or helper with the
 * HIP library.
 *
 * Every function takes fp64 arrays (the exact upcast of whatever the caller
 * stored), contiguous and row-major with the last index fastest, and returns
 * 0 on success or -1 on a bad argument. Optional inputs are NULL when absent:
 *   Dskip NULL -> no skip term;  z NULL -> no gate;  h0 NULL -> zero state;
 *   h_final NULL -> not written.
 *
 * Layouts (Mamba-1):  x, delta, z, y [B,L,D]; Bm, Cm [B,L,N]; A [D,N];
 *                     Dskip [D]; h0, h_final [B,D,N].
 * Layouts (SSD):      x, z, y [B,L,H,P]; delta [B,L,H]; A [H]; Bm, Cm [B,L,N];
 *                     Dskip [H]; h0, h_final [B,H,N,P].
 * Layouts (step):     state [B,D,N] (updated in place); x, delta, z, y [B,D];
 *                     Bm, Cm [B,N]; A [D,N]; Dskip [D].
 */
#ifndef SSM_ORACLE_H
#define SSM_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Number of OpenMP threads the oracle uses (n <= 0 restores the default). */
void oracle_set_threads(int n);
int oracle_get_threads(void);

/* O1: Mamba-1 selective scan, one time step after another. */
int oracle_scan(int B, int L, int D, int N,
                const double* x, const double* delta, const double* A,
                const double* Bm, const double* Cm, const double* Dskip,
                const double* z, const double* h0, double* y, double* h_final);

/* O2: Mamba-2 (SSD) recurrence with a scalar decay per head, sequential. */
int oracle_ssd_seq(int B, int L, int H, int P, int N,
                   const double* x, const double* delta, const double* A,
                   const double* Bm, const double* Cm, const double* Dskip,
                   const double* z, const double* h0, double* y, double* h_final);

/* O3: SSD in chunked (decayed-attention) form with chunk length Q >= 1. */
int oracle_ssd_chunked(int B, int L, int H, int P, int N, int Q,
                       const double* x, const double* delta, const double* A,
                       const double* Bm, const double* Cm, const double* Dskip,
                       const double* z, const double* h0, double* y, double* h_final);

/* O4: one recurrent decode step; state is read and written in place. */
int oracle_step(int B, int D, int N, double* state,
                const double* x, const double* delta, const double* A,
                const double* Bm, const double* Cm, const double* Dskip,
                const double* z, double* y);

/* O4': one SSD decode step (scalar decay per head); state [B,H,N,P] in place;
 * x, z, y [B,H,P]; delta [B,H]; Bm, Cm [B,N]; A, Dskip [H]. */
int oracle_ssd_step(int B, int H, int P, int N, double* state,
                    const double* x, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, double* y);

/* O5: brute-force unrolled state (O(L^2) explicit products), tiny shapes. */
int oracle_scan_unroll(int B, int L, int D, int N,
                       const double* x, const double* delta, const double* A,
                       const double* Bm, const double* Cm, const double* Dskip,
                       const double* z, const double* h0, double* y, double* h_final);

int oracle_ssd_unroll(int B, int L, int H, int P, int N,
                      const double* x, const double* delta, const double* A,
                      const double* Bm, const double* Cm, const double* Dskip,
                      const double* z, const double* h0, double* y, double* h_final);

/* O6: gradient of O1 (training backward pass). For the loss
 * l = sum(dy * y) + sum(dh_final * h_final) it writes dl/d(input) for every
 * input: dx, ddelta, dz [B,L,D]; dA [D,N]; dBm, dCm [B,L,N]; dDskip [D];
 * dh0 [B,D,N]. dy [B,L,D] is required; dh_final [B,D,N] may be NULL (zero).
 * dDskip is written when Dskip is given, dz when z is given; dh0 may be NULL. */
int oracle_scan_bwd(int B, int L, int D, int N,
                    const double* x, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, const double* h0,
                    const double* dy, const double* dh_final,
                    double* dx, double* ddelta, double* dA, double* dBm, double* dCm,
                    double* dDskip, double* dz, double* dh0);

/* O7: O1 and O4 with a choice of discretisation and Delta preprocessing:
 * disc 0 = exponential-Euler (Bbar = Delta B), 1 = exact zero-order hold
 * (Bbar = Delta B (e^z - 1)/z, z = Delta A; Taylor 1 + z/2 + z^2/6 for |z| < 1e-4);
 * Delta = softplus(delta + delta_bias[d]) when delta_softplus is set (the bias
 * is added first whenever delta_bias is not NULL). */
int oracle_scan_disc(int B, int L, int D, int N, int disc, const double* delta_bias, int delta_softplus,
                     const double* x, const double* delta, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     const double* z, const double* h0, double* y, double* h_final);

int oracle_step_disc(int B, int D, int N, int disc, const double* delta_bias, int delta_softplus,
                     double* state, const double* x, const double* delta, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     const double* z, double* y);

/* O8: Mamba-3 selective scan with complex diagonal transitions and the
 * exponential-trapezoidal rule. Per (b, d), complex state h[n], for t = 0..L-1:
 *   alpha = exp(delta_t * (Are[d,n] + i theta[d,n]))
 *   h[n]  = alpha h[n] + (1 - lam_t) delta_t alpha B_{t-1}[n] x_{t-1} + lam_t delta_t B_t[n] x_t
 *   y_t   = (sum_n C_t[n] Re(h[n]) + D x_t) silu(z_t)
 * with B_{-1} x_{-1} taken from x_prev [B,D] and B_prev [B,N] (both NULL: zero).
 * h0 and h_final are complex, [B,D,N,2] (real, imaginary); h0 NULL = zero.
 * lam = 1, theta = 0 is exactly O1's exponential-Euler recurrence. */
int oracle_scan3(int B, int L, int D, int N,
                 const double* x, const double* delta, const double* lam,
                 const double* Are, const double* theta,
                 const double* Bm, const double* Cm, const double* Dskip, const double* z,
                 const double* h0, const double* x_prev, const double* B_prev,
                 double* y, double* h_final);

#ifdef __cplusplus
}
#endif
#endif
