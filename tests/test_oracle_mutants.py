"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutant is a one-spot text edit of ``oracle/oracle.c`` (a dropped term, a
wrong sign or index, a transposed operand, an off-by-one decay), compiled into a
throw-away library. The test passes when at least one pin fails on it.
"""
import os

import pytest

import oracle
from oracle import build as obuild
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "scan_decay_sign": ("abar = exp(dt * A[d * N + n]); /*", "abar = exp(-dt * A[d * N + n]); /*"),
    "scan_drop_delta_in_input": ("h[n] = abar * h[n] + dt * Bt[n] * xv;", "h[n] = abar * h[n] + Bt[n] * xv;"),
    "scan_C_swapped_for_B": ("ch += Ct[n] * h[n];", "ch += Bt[n] * h[n];"),
    "scan_output_before_update": ("abar = exp(dt * A[d * N + n]); /* exponential-Euler */\n                h[n] = abar * h[n] + dt * Bt[n] * xv;\n                ch += Ct[n] * h[n];",
                                  "abar = exp(dt * A[d * N + n]); /* exponential-Euler */\n                ch += Ct[n] * h[n];\n                h[n] = abar * h[n] + dt * Bt[n] * xv;"),
    "scan_A_index_transposed": ("abar = exp(dt * A[d * N + n]); /* exponential-Euler */", "abar = exp(dt * A[n * D + d]); /* exponential-Euler */"),
    "skip_term_dropped": ("if (Dskip) v += Dskip[dix] * xv;", ""),
    "gate_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "ssd_seq_wrong_head_decay": ("double abar = exp(dt * A[hh]);\n            const double* Bt", "double abar = exp(dt * A[0]);\n            const double* Bt"),
    "ssd_seq_state_transposed": ("ch += Ct[n] * S[n * P + p];\n                long i", "ch += Ct[n] * S[p * N + n];\n                long i"),
    "ssd_chunk_exclusive_prefix": ("acc += delta[(b * L + c0 + i) * H + hh] * A[hh];\n                s[i] = acc;",
                                   "s[i] = acc;\n                acc += delta[(b * L + c0 + i) * H + hh] * A[hh];"),
    "ssd_chunk_no_offdiag_decay": ("yo *= exp(s[i]);", ""),
    "ssd_chunk_no_state_decay": ("double v = exp(slast) * S[n * P + p];", "double v = S[n * P + p];"),
    "ssd_chunk_strict_causal": ("for (int j = 0; j <= i; ++j) {\n                        long tj", "for (int j = 0; j < i; ++j) {\n                        long tj"),
    "ssd_chunk_G_transposed": ("g += Cm[(b * L + c0 + i) * N + n] * Bm[(b * L + c0 + j) * N + n];",
                               "g += Cm[(b * L + c0 + j) * N + n] * Bm[(b * L + c0 + i) * N + n];"),
    "step_no_decay": ("h[n] = exp(dt * A[d * N + n]) * h[n] + dt * Bm[b * N + n] * xv;", "h[n] = h[n] + dt * Bm[b * N + n] * xv;"),
    "ssd_step_no_delta": ("S[n * P + p] = abar * S[n * P + p] + dt * Bm[b * N + n] * xt[p];", "S[n * P + p] = abar * S[n * P + p] + Bm[b * N + n] * xt[p];"),
    "hfinal_not_written": ("h_final[(b * D + d) * N + n] = h[n];", "h_final[(b * D + d) * N + n] = 0.0;"),
    "bwd_adjoint_no_decay": ("c[n] = abar * g;", "c[n] = g;"),
    "bwd_dA_uses_current_state": ("dA[d * N + n] += g * abar * hprev[n] * dt;", "dA[d * N + n] += g * abar * hcur[n] * dt;"),
    "bwd_ddelta_drops_input_term": ("gdt += g * (A[d * N + n] * abar * hprev[n] + Bt[n] * xv);",
                                    "gdt += g * (A[d * N + n] * abar * hprev[n]);"),
    "bwd_dz_drops_sigmoid_slope": ("dz[i] = dy[i] * v * s * (1.0 + z[i] * (1.0 - s));", "dz[i] = dy[i] * v * s;"),
    "bwd_dB_drops_delta": ("pB[(b * L + t) * N + n] += g * dt * xv;", "pB[(b * L + t) * N + n] += g * xv;"),
    "bwd_dC_uses_adjoint": ("pC[(b * L + t) * N + n] += dv * hcur[n];", "pC[(b * L + t) * N + n] += g * hcur[n];"),
    "bwd_skip_gradient_ungated": ("gx = dv * Dskip[d];", "gx = dy[i] * Dskip[d];"),
    "bwd_adjoint_ignores_dh_final": ("c[n] = dh_final ? dh_final[(b * D + d) * N + n] : 0.0;", "c[n] = 0.0;"),
    "bwd_dx_uses_C": ("gx += g * dt * Bt[n];", "gx += g * dt * Ct[n];"),
    "zoh_taylor_sign": ("return 1.0 + z / 2.0 + z * z / 6.0;", "return 1.0 - z / 2.0 + z * z / 6.0;"),
    "zoh_exact_branch_not_divided": ("return (exp(z) - 1.0) / z;", "return (exp(z) - 1.0);"),
    "zoh_coefficient_without_delta": ("*bcoef = disc == 1 ? dt * zoh_phi(dt * a) : dt;",
                                      "*bcoef = disc == 1 ? zoh_phi(dt * a) : dt;"),
    "delta_bias_ignored": ("if (delta_bias) dt += delta_bias[d];", ""),
    "softplus_large_branch_truncated": ("return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));",
                                        "return v > 0.0 ? v : log1p(exp(v));"),
    "m3_prev_term_without_decay": ("(1.0 - lm) * dt * alpha * prev", "(1.0 - lm) * dt * prev"),
    "m3_lambda_weights_swapped": ("(1.0 - lm) * dt * alpha * prev + lm * dt * Bt[n] * xv",
                                  "lm * dt * alpha * prev + (1.0 - lm) * dt * Bt[n] * xv"),
    "m3_rotation_sign": ("cexp(dt * (Are[d * N + n] + I * theta[d * N + n]))",
                         "cexp(dt * (Are[d * N + n] - I * theta[d * N + n]))"),
    "m3_output_reads_imaginary_part": ("ch += Ct[n] * creal(h[n]);", "ch += Ct[n] * cimag(h[n]);"),
    "m3_previous_token_not_advanced": ("xp = xv;\n            Bp = Bt;", "Bp = Bt;"),
    "m3_h0_imaginary_dropped": ("h[n] = h0 ? h0[k] + I * h0[k + 1] : 0.0;", "h[n] = h0 ? h0[k] : 0.0;"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "oracle.c"
    src.write_text(source.replace(old, new))
    (tmp_path / "oracle.h").write_text(open(os.path.join(os.path.dirname(SRC), "oracle.h")).read())
    lib = obuild.build(src=str(src), out=str(tmp_path / f"lib_{name}.so"), quiet=True)
    mut = oracle.Oracle(lib)
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(mut)
        except (AssertionError, ValueError, FloatingPointError) as e:
            failures.append(pin.__name__)
    assert failures, f"no pin caught the planted mistake {name}"
