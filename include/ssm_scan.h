/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective state-space scan library.
 *
 * Entry points, each a hand-written HIP kernel pipeline for CDNA4:
 *   ssm_scan_fwd     Mamba-1 selective scan over a whole sequence (prefill)
 *   ssm_scan_fwd_noalloc  the same on a fixed per-GPU scratch (no workspace argument)
 *   ssm_scan_fwd_ex  the same with exact zero-order hold and/or Delta = softplus(delta + bias)
 *   ssm_scan3_fwd    Mamba-3: complex transitions, exponential-trapezoidal rule
 *   ssm_step3        the Mamba-3 one-token decode step, complex state updated in place
 *   ssm_scan_bwd     the scan's gradient (training backward pass)
 *   ssm_ssd_fwd      Mamba-2 SSD: scalar decay per head, chunked decayed-attention form
 *   ssm_step         one-token recurrent decode step, state updated in place
 *   ssm_step_ex      the decode step with the options of ssm_scan_fwd_ex
 *   ssm_ssd_step     the same for the Mamba-2 form (scalar decay per head, (N, P) state)
 *
 * The operation (selective SSM of Gu & Dao, "Mamba: Linear-Time Sequence
 * Modeling with Selective State Spaces", 2023, and the SSD form of Dao & Gu,
 * "Transformers are SSMs", 2024 -- both in the ssm-bench README's references;
 * the variants as described by "Efficient Sequence Modeling: From S4 to
 * Mamba-3", section 03 System: mamba_minimal.py has input-dependent Delta, B, C
 * and an incremental step(); mamba2_minimal.py has a scalar A per head, chunked
 * decayed-attention matmuls and a carried (N, P) state):
 *
 *   per (batch b, channel d), state h in R^N, for t = 0 .. L-1:
 *     h_t = exp(Delta_t * A) (.) h_{t-1} + Delta_t * B_t * x_t      (exponential-Euler:
 *     y_t = (C_t . h_t + D * x_t) * silu(z_t),  silu(z) = z / (1 + e^-z)   section 04/09)
 *
 * Conventions shared by every entry point
 *  - Tensors are contiguous, row-major, last index fastest.
 *  - Every pointer is a DEVICE pointer owned by the caller. The library never
 *    allocates, frees or synchronises inside these calls and keeps no pointer
 *    after return, except for work in flight on `stream`.
 *  - `stream` is a hipStream_t (NULL = the default stream). All work is queued
 *    asynchronously on it; results are ready when the stream reaches that point.
 *  - `io` (ssm_dtype_t) is the storage type of x, delta, B, C, z and y.
 *    A, D, h0, h_final and the decode state are always fp32.
 *    Arithmetic is fp32 throughout (fp32 state and accumulation).
 *  - delta is used as given (already positive: no softplus inside).
 *  - A holds the actual (negative) decay rates, not log(-A).
 *  - B and C are one group shared by all channels (Mamba-1) or all heads (SSD).
 *  - Optional pointers may be NULL: Dskip (no skip term), z (no gate),
 *    h0 (zero initial state), h_final (not written).
 *  - Aliasing: y must not alias any input; h_final must not alias h0.
 *  - Errors: arguments are validated BEFORE any HIP call. A rejected call has
 *    queued nothing. Status codes are below; ssm_last_error() returns a
 *    human-readable detail of the calling thread's last failure.
 *    No C++ exception crosses this boundary.
 *  - Results are deterministic run to run (no floating-point atomics).
 *  - Thread-safe and reentrant: no mutable global state beyond a per-thread
 *    error message and cached device properties.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 1

/* Storage type of the io tensors. The last enumerator only widens the type to a
 * full int, so any int a caller passes is a valid value (out-of-range values are
 * rejected with SSM_ERR_INVALID_ARG). */
typedef enum { SSM_F32 = 0, SSM_BF16 = 1, SSM_DTYPE_INT_RANGE_ = 0x7fffffff } ssm_dtype_t;

/* Discretisation of the continuous system dh/dt = A h + B x over one step Delta
 * (diagonal A). Exponential-Euler is what every entry point uses by default. */
typedef enum {
    SSM_DISC_EULER = 0, /* Abar = exp(Delta A), Bbar = Delta B */
    SSM_DISC_ZOH = 1,   /* Abar = exp(z), Bbar = Delta B (e^z - 1)/z, z = Delta A (exact zero-order hold) */
    SSM_DISC_INT_RANGE_ = 0x7fffffff
} ssm_disc_t;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_INVALID_ARG = 1, /* null required pointer, bad dimension, misaligned pointer */
    SSM_ERR_UNSUPPORTED = 2, /* shape outside the compiled range (e.g. unsupported N or P) */
    SSM_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than *_workspace_size() */
    SSM_ERR_HIP = 4          /* a HIP launch error (hipGetLastError after the launch) */
} ssm_status_t;

/* SSM_ABI_VERSION of the built library. */
int ssm_abi_version(void);

/* Static string naming a status code. */
const char* ssm_status_string(int status);

/* Detail of the calling thread's last non-OK status ("" if none). */
const char* ssm_last_error(void);

/* Kernel-level timing without a profiler (diagnostic; for benchmarks).
 * After ssm_profile_events(events, n) with n > 0, every kernel launched by an
 * entry point called from this thread takes the next two events (events[0] and
 * events[1] for the first kernel, and so on; each a hipEvent_t created by the
 * caller), which the HIP runtime stamps at that kernel's own start and end
 * (hipExtLaunchKernel), so hipEventElapsedTime of a pair is the kernel's
 * duration. Recording stops when fewer than two events remain.
 * ssm_profile_events(NULL, 0) switches recording off. Returns the number of
 * events used since the previous call (twice the number of kernels timed).
 * Per thread; the library never creates, synchronises or destroys the events. */
int ssm_profile_events(void* const* events, int n);

/* ---------------------------------------------------------------------------
 * ssm_scan_fwd -- Mamba-1 selective scan (prefill).
 *
 * Defined by "Efficient Sequence Modeling: From S4 to Mamba-3", section 03
 * System (mamba_minimal.py: input-dependent Delta, B, C and an explicit
 * time-loop selective scan), with the exponential-Euler discretisation the
 * same page names as the lambda = 1, theta = 0 limit (section 04, "Complex
 * transitions for state tracking"; section 09 Validation). Per (b, d), over
 * t = 0 .. L-1, from h = h0[b, d, :] (or zeros):
 *   h[n]      = exp(delta[b,t,d] * A[d,n]) * h[n] + delta[b,t,d] * Bm[b,t,n] * x[b,t,d]
 *   y[b,t,d]  = (sum_n Cm[b,t,n] * h[n] + Dskip[d] * x[b,t,d]) * silu(z[b,t,d])
 *   h_final[b, d, :] = h after the last step.
 * The work is cut along L into segments whose carried states compose as affine
 * maps; the result equals the sequential recurrence up to rounding.
 *
 *   x, delta, z, y : [B, L, D]  io dtype     (z may be NULL)
 *   A              : [D, N]     fp32, A < 0 as used in exp(delta * A)
 *   Bm, Cm         : [B, L, N]  io dtype, shared by all D channels
 *   Dskip          : [D]        fp32 or NULL
 *   h0             : [B, D, N]  fp32 or NULL (zeros)
 *   h_final        : [B, D, N]  fp32 out, or NULL
 *   workspace      : device scratch of at least ssm_scan_workspace_size(B, L, D, N)
 *                    bytes (NULL allowed when that size is 0); contents on entry
 *                    are ignored and on return are undefined.
 * Supported: N in {4, 8, 16, 32, 64, 128, 256}; B, D >= 1; L >= 0 (L = 0 writes
 * h_final = h0). N = 256 needs a workspace whenever L > 0 (it holds the C . h sums
 * of its two groups of state chunks).
 * Every pointer must be 16-byte aligned.
 * ------------------------------------------------------------------------- */
size_t ssm_scan_workspace_size(int B, int L, int D, int N);

int ssm_scan_fwd(int B, int L, int D, int N, ssm_dtype_t io,
                 const void* x, const void* delta, const float* A,
                 const void* Bm, const void* Cm, const float* Dskip,
                 const void* z, const float* h0,
                 void* y, float* h_final,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ssm_scan_fwd_noalloc -- ssm_scan_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no workspace argument, and nothing is allocated or freed.
 *
 * The scan's carry workspace is a fixed device array inside the library,
 * SSM_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, held from the library's load until
 * the process ends. Its device address is looked up on the first call made for
 * a device (with that device made current for the lookup). Every other argument,
 * the result and the errors are those of ssm_scan_fwd; a shape whose
 * ssm_scan_workspace_size() exceeds SSM_NOALLOC_SCRATCH_BYTES returns
 * SSM_ERR_UNSUPPORTED (for instance B=8, L=32768, D=512, N=16 needs 99.5 MiB
 * and fits; N = 256 at B=1, L=4096, D=1536 needs 141.2 MiB and does not). The
 * kernels run on the device of `stream` (the current device when stream is NULL).
 *
 * Concurrency: all calls on one GPU share its scratch array and nothing clears
 * it between calls (the scan ignores its previous contents). Calls that can
 * overlap on one GPU -- on different streams, or from different threads without
 * ordering -- race on it and give undefined results; serialise them (one stream,
 * or events between streams).
 * ------------------------------------------------------------------------- */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

int ssm_scan_fwd_noalloc(int B, int L, int D, int N, ssm_dtype_t io,
                         const void* x, const void* delta, const float* A,
                         const void* Bm, const void* Cm, const float* Dskip,
                         const void* z, const float* h0,
                         void* y, float* h_final, void* stream);

/* ---------------------------------------------------------------------------
 * ssm_scan_fwd_ex -- ssm_scan_fwd with a choice of discretisation and the
 * Delta preprocessing done inside the kernels.
 *
 *   disc           SSM_DISC_EULER or SSM_DISC_ZOH. Exact zero-order hold is the
 *                  discretisation of "Efficient Sequence Modeling: From S4 to
 *                  Mamba-3" (section 03, s4_minimal.py; section 04 "Math-verified
 *                  discretization"; Q01): Bbar = Delta B (e^z - 1)/z, z = Delta A,
 *                  evaluated without the 0/0 at z = 0 (a series where |z| < 1/32).
 *   delta_bias     [D] fp32 or NULL: added to delta before everything else.
 *   delta_softplus nonzero: Delta = softplus(delta + delta_bias) = log(1 + e^(.)).
 * Every other argument, the workspace (ssm_scan_workspace_size) and the errors
 * are those of ssm_scan_fwd; with SSM_DISC_EULER, no bias and no softplus it is
 * ssm_scan_fwd. Every N of ssm_scan_fwd is supported (N >= 64 runs as chunks of
 * 16 states, as there). delta_bias must be 16-byte aligned.
 * ------------------------------------------------------------------------- */
int ssm_scan_fwd_ex(int B, int L, int D, int N, ssm_dtype_t io, ssm_disc_t disc,
                    const float* delta_bias, int delta_softplus,
                    const void* x, const void* delta, const float* A,
                    const void* Bm, const void* Cm, const float* Dskip,
                    const void* z, const float* h0,
                    void* y, float* h_final,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ssm_scan3_fwd -- Mamba-3 selective scan: complex diagonal transitions and the
 * exponential-trapezoidal rule.
 *
 * "Efficient Sequence Modeling: From S4 to Mamba-3", section 03 System
 * (mamba3_minimal.py: complex diagonal transitions A = -exp(a) + i theta with a
 * data-dependent exponential-trapezoidal rule, reducing to Mamba-1/2 at lam = 1)
 * and section 04 "Complex transitions for state tracking" (the rotation phase
 * lets the state track parity; lam = 1, theta = 0 is exponential-Euler). The
 * pages do not write the rule out; the reading implemented is the trapezoidal
 * rule, weighted by lam, on the exact one-step integral of e^{A (Delta - s)} B x.
 * Per (b, d), complex state h[n], for t = 0 .. L-1:
 *   alpha   = exp(delta[b,t,d] * (Are[d,n] + i theta[d,n]))
 *   h[n]    = alpha h[n] + (1 - lam[b,t,d]) delta[b,t,d] alpha Bm[b,t-1,n] x[b,t-1,d]
 *                        + lam[b,t,d] delta[b,t,d] Bm[b,t,n] x[b,t,d]
 *   y[b,t,d] = (sum_n Cm[b,t,n] Re(h[n]) + Dskip[d] x[b,t,d]) * silu(z[b,t,d])
 * where the step before t = 0 is (x_prev[b,d], B_prev[b,:]) -- the last token of
 * a previous call, so that a sequence can be continued -- or zero when both are
 * NULL.
 *
 *   x, delta, lam, z, y : [B, L, D]  io dtype (z may be NULL); lam in [0, 1]
 *   Are, theta     : [D, N]     fp32 (Are < 0: the real part of A; theta in radians
 *                               per unit of delta)
 *   Bm, Cm         : [B, L, N]  io dtype
 *   Dskip          : [D]        fp32 or NULL
 *   h0, h_final    : [B, D, N, 2] fp32 complex (real, imaginary), or NULL
 *   x_prev, B_prev : [B, D], [B, N] io dtype, both given or both NULL
 *   workspace      : at least ssm_scan3_workspace_size(B, L, D, N) bytes
 * Supported: N in {4, 8, 16}; B <= 65535. Every pointer must be 16-byte aligned.
 * Errors as for ssm_scan_fwd.
 * ------------------------------------------------------------------------- */
size_t ssm_scan3_workspace_size(int B, int L, int D, int N);

int ssm_scan3_fwd(int B, int L, int D, int N, ssm_dtype_t io,
                  const void* x, const void* delta, const void* lam,
                  const float* Are, const float* theta,
                  const void* Bm, const void* Cm, const float* Dskip, const void* z,
                  const float* h0, const void* x_prev, const void* B_prev,
                  void* y, float* h_final,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ssm_step3 -- Mamba-3 one-token decode step: the recurrence of ssm_scan3_fwd for
 * one time step, the complex state updated in place.
 *
 * "Efficient Sequence Modeling: From S4 to Mamba-3", section 03 System
 * (mamba3_minimal.py: the incremental form of the complex, exponential-trapezoidal
 * recurrence). Per (batch b, channel d) and state n:
 *   alpha = exp(delta (Are[d,n] + i theta[d,n]))
 *   h[n]  = alpha (h[n] + (1 - lam) delta B_prev[n] x_prev) + lam delta B[n] x
 *   y     = (sum_n C[n] Re h[n] + Dskip[d] x) * silu(z)
 * ssm_step3 on a state equals ssm_scan3_fwd over one token from that state with
 * the same (x_prev, B_prev); a decode loop passes the previous token's x and B
 * row as the next call's x_prev and B_prev.
 *
 *   state  : [B, D, N, 2] fp32 (real, imaginary), read and written in place
 *   x, delta, lam, z : [B, D] io dtype (z may be NULL: no gate)
 *   Are, theta       : [D, N] fp32, as for ssm_scan3_fwd
 *   Bm, Cm           : [B, N] io dtype
 *   Dskip            : [D] fp32 or NULL
 *   x_prev, B_prev   : [B, D] and [B, N] io dtype, both or neither (neither: the
 *                      previous token's term is zero, as at a sequence start)
 *   y                : [B, D] io dtype out
 * Supported: N in {4, 8, 16, 32, 64, 128}; B <= 65535; D * N < 2^31. Every pointer
 * must be 16-byte aligned. Errors: SSM_ERR_INVALID_ARG (a required pointer NULL,
 * x_prev without B_prev or the reverse, bad dims, misalignment), SSM_ERR_UNSUPPORTED
 * (N, B or D * N out of range), SSM_ERR_HIP.
 * ------------------------------------------------------------------------- */
int ssm_step3(int B, int D, int N, ssm_dtype_t io,
              float* state, const void* x, const void* delta, const void* lam,
              const float* Are, const float* theta, const void* Bm, const void* Cm,
              const float* Dskip, const void* z, const void* x_prev, const void* B_prev,
              void* y, void* stream);

/* ---------------------------------------------------------------------------
 * ssm_scan_bwd -- gradient of ssm_scan_fwd (training backward pass).
 *
 * Training Mamba models on GPUs is the workload of "Characterizing the Behavior
 * of Training Mamba-based State Space Models on GPUs" (abstract) and of the
 * training-step sweep in "Efficient Sequence Modeling: From S4 to Mamba-3",
 * section 05 Evaluation. The pages do not write the backward pass out: this is
 * the exact gradient of the forward recurrence above, by the chain rule. For
 * the loss  l = sum(dy * y) + sum(dh_final * h_final)  every output is dl/d(the
 * input of the same name):
 *
 *   inputs  : x, delta, A, Bm, Cm, Dskip, z, h0 exactly as given to ssm_scan_fwd
 *   dy      : [B, L, D]  io dtype, gradient of y (required)
 *   dh_final: [B, D, N]  fp32 gradient of h_final, or NULL (zero)
 *   dx, ddelta : [B, L, D] io dtype out
 *   dA      : [D, N]     fp32 out (summed over batch and time)
 *   dBm, dCm: [B, L, N]  io dtype out (summed over channels in fp32, then rounded)
 *   dDskip  : [D]        fp32 out; given exactly when Dskip is given
 *   dz      : [B, L, D]  io dtype out; given exactly when z is given
 *   dh0     : [B, D, N]  fp32 out, or NULL (not written); the gradient of the
 *                        initial state, also when h0 is NULL (zero state)
 *   workspace: device scratch of at least ssm_scan_bwd_workspace_size(B, L, D, N)
 *              bytes (0 only when L = 0); contents on entry are ignored.
 * The forward states are recomputed, not read from a forward call. Outputs must
 * not alias inputs or each other. Arithmetic is fp32 with fp32 accumulation;
 * reductions run in a fixed order (no atomics), so results are deterministic.
 * Supported: N in {4, 8, 16, 32, 64, 128, 256} (N >= 32 runs as chunks of 16
 * states whose partial sums over n are added in a fixed order: chunk order within
 * groups of up to four chunks, then the groups in order); B <= 65535; L >= 0
 * (L = 0 writes dh0 = dh_final, dA = 0, dDskip = 0). Every pointer must be
 * 16-byte aligned. Errors as for ssm_scan_fwd.
 * ------------------------------------------------------------------------- */
size_t ssm_scan_bwd_workspace_size(int B, int L, int D, int N);

int ssm_scan_bwd(int B, int L, int D, int N, ssm_dtype_t io,
                 const void* x, const void* delta, const float* A,
                 const void* Bm, const void* Cm, const float* Dskip,
                 const void* z, const float* h0,
                 const void* dy, const float* dh_final,
                 void* dx, void* ddelta, float* dA, void* dBm, void* dCm,
                 float* dDskip, void* dz, float* dh0,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ssm_ssd_fwd -- Mamba-2 SSD chunked scan (prefill), scalar decay per head.
 *
 * Defined by "Efficient Sequence Modeling: From S4 to Mamba-3", section 03
 * System (mamba2_minimal.py: a scalar A per head reduces the recurrence to SSD,
 * computed as chunked decayed-attention matmuls with a carried (N, P) state)
 * and section 04 "Chunked SSD with a sequential reference" (the chunked form
 * equals the sequential recurrence). Per (b, h), from S = h0[b, h] (or zeros):
 *   S[n, p]    = exp(delta[b,t,h] * A[h]) * S[n, p] + delta[b,t,h] * Bm[b,t,n] * x[b,t,h,p]
 *   y[b,t,h,p] = (sum_n Cm[b,t,n] * S[n, p] + Dskip[h] * x[b,t,h,p]) * silu(z[b,t,h,p])
 *   h_final[b, h] = S after the last step.
 * Inside a chunk, with s_i the inclusive prefix of delta * A_h:
 *   y_i = sum_{j <= i} (C_i . B_j) exp(s_i - s_j) delta_j x_j + exp(s_i) C_i S_in (+ skip, gate);
 *   S_out = exp(s_last) S_in + sum_j exp(s_last - s_j) delta_j B_j^T x_j.
 *
 *   x, z, y : [B, L, H, P]  io dtype     (z may be NULL)
 *   delta   : [B, L, H]     io dtype
 *   A       : [H]           fp32, A_h < 0
 *   Bm, Cm  : [B, L, N]     io dtype, one group shared by all H heads
 *   Dskip   : [H]           fp32 or NULL
 *   h0      : [B, H, N, P]  fp32 or NULL (zeros)
 *   h_final : [B, H, N, P]  fp32 out, or NULL
 *   chunk   : chunk length Q >= 1 (0 = default 256). The last chunk is ragged
 *             when Q does not divide L. The result does not depend on Q beyond
 *             rounding; chunks above 256 steps run as 256-step chunks (one
 *             chunk's rows must fit a workgroup's LDS). The kernels tile a chunk
 *             by 32 rows, so a chunk that is not a multiple of 32 costs the work
 *             of the next multiple.
 * Supported: io = SSM_BF16; N in {64, 128}; P = 64; B, H <= 65535;
 * B * H <= 2^24; L * H * P * 2 < 2^31.
 * ------------------------------------------------------------------------- */
size_t ssm_ssd_workspace_size(int B, int L, int H, int P, int N, int chunk);

int ssm_ssd_fwd(int B, int L, int H, int P, int N, int chunk, ssm_dtype_t io,
                const void* x, const void* delta, const float* A,
                const void* Bm, const void* Cm, const float* Dskip,
                const void* z, const float* h0,
                void* y, float* h_final,
                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * ssm_step -- one-token recurrent decode step, state read and written in place.
 *
 * Defined by "Efficient Sequence Modeling: From S4 to Mamba-3", section 03
 * System (mamba_minimal.py's incremental step() for decoding) and section 09
 * Validation (step() equals a full forward): one iteration of the ssm_scan_fwd
 * recurrence above, per (b, d), on the state [b, d, :] held in place.
 *
 *   state  : [B, D, N]  fp32, updated in place
 *   x, delta, z, y : [B, D]  io dtype   (z may be NULL)
 *   A      : [D, N]  fp32
 *   Bm, Cm : [B, N]  io dtype
 *   Dskip  : [D]     fp32 or NULL
 * Supported: N in {4, 8, 16, 32, 64, 128, 256}; B <= 65535; D * N <= 2^32.
 * ------------------------------------------------------------------------- */
int ssm_step(int B, int D, int N, ssm_dtype_t io,
             float* state, const void* x, const void* delta, const float* A,
             const void* Bm, const void* Cm, const float* Dskip, const void* z,
             void* y, void* stream);

/* ssm_step_ex -- ssm_step with disc, delta_bias and delta_softplus as in
 * ssm_scan_fwd_ex (all N of ssm_step), so a sequence prefilled with
 * ssm_scan_fwd_ex continues token by token with the same options. */
int ssm_step_ex(int B, int D, int N, ssm_dtype_t io, ssm_disc_t disc,
                const float* delta_bias, int delta_softplus,
                float* state, const void* x, const void* delta, const float* A,
                const void* Bm, const void* Cm, const float* Dskip, const void* z,
                void* y, void* stream);

/* ---------------------------------------------------------------------------
 * ssm_ssd_step -- one-token decode step of the Mamba-2 form, state in place
 * (the incremental step of "Efficient Sequence Modeling: From S4 to Mamba-3",
 * section 03, applied to mamba2_minimal.py's per-head scalar decay and (N, P)
 * state). Per batch b and head h, with a = exp(delta[b,h] * A[h]):
 *   S[n, p] = a * S[n, p] + delta[b,h] * Bm[b,n] * x[b,h,p]
 *   y[b,h,p] = (sum_n Cm[b,n] * S[n, p] + Dskip[h] * x[b,h,p]) * silu(z[b,h,p])
 *
 *   state  : [B, H, N, P]  fp32, updated in place
 *   x, z, y : [B, H, P]    io dtype   (z may be NULL)
 *   delta  : [B, H]        io dtype
 *   A      : [H]           fp32
 *   Bm, Cm : [B, N]        io dtype, shared by all heads
 *   Dskip  : [H]           fp32 or NULL
 * Supported: P = 64; N in {16, 32, 64, 128, 256}; B * H <= 2^31 - 1.
 * Errors as for ssm_step; every pointer must be 16-byte aligned.
 * ------------------------------------------------------------------------- */
int ssm_ssd_step(int B, int H, int P, int N, ssm_dtype_t io,
                 float* state, const void* x, const void* delta, const float* A,
                 const void* Bm, const void* Cm, const float* Dskip, const void* z,
                 void* y, void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostics for benchmarks (not part of the method; asynchronous on `stream`,
 * time them with events on that stream).
 *
 * ssm_diag_valu_rate: `blocks` workgroups of 256 lanes, each lane running 8
 *   independent chains for `iters` rounds of 4 dependent ops: mode 0 v_exp_f32
 *   only, mode 1 v_fma_f32 only, mode 2 one v_exp_f32 per three v_fma_f32, mode 3
 *   v_sin_f32 only, mode 4 v_cos_f32 only (so blocks * 256 * 32 * iters ops in
 *   all). out: blocks * 256 floats (a sum per lane, so nothing is optimised away).
 * ssm_diag_stream_scale: p[i] *= s for i < n, in place (n a multiple of 4): what a
 *   kernel that only reads and writes an array of the decode state's size reaches.
 * ssm_diag_copy: dst[i] = src[i] (n a multiple of 4): the byte reference that
 *   scales HBM byte counters.
 * Pointers are device pointers, 16-byte aligned. Errors as for the entry points.
 * ------------------------------------------------------------------------- */
int ssm_diag_valu_rate(int mode, int blocks, int iters, float* out, void* stream);
int ssm_diag_stream_scale(float* p, size_t n, float s, void* stream);
int ssm_diag_copy(const float* src, float* dst, size_t n, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_SCAN_H */
