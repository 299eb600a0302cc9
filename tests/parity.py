"""Parity metric between a GPU result and the fp64 oracle.

Tolerance: relative error <= 1e-3 (fp32 arithmetic, bf16/fp32 storage).
Two checks, both must pass:

* element by element, in the form the "From S4 to Mamba-3" case study uses for
  its equivalence tests (allclose with atol = rtol = 1e-3, section 04/09), with
  the absolute part scaled to the tensor (1e-3 * rms of the oracle values) and
  with half a storage ulp added, since a bf16-stored output cannot be closer
  to the fp64 value than its own rounding:
      |g - r| <= 0.5 ulp_storage(max(|g|, |r|)) + 1e-3 * |r| + 1e-3 * rms(r)
* normwise: ||g - r|| / ||r|| <= 1e-3 for fp32-stored tensors; for bf16-stored
  tensors the excess over the unavoidable storage rounding,
  sqrt(max(0, err^2 - q^2)) with q = ||bf16(r) - r|| / ||r||, must be <= 1e-3.
"""
import numpy as np

import ssm_inputs as si

REL_TOL = 1e-3


def half_ulp(v, storage):
    a = np.abs(v)
    m, e = np.frexp(np.where(a > 0, a, 1.0))      # a = m 2^e, m in [0.5, 1)
    mant_bits = 8 if storage == "bf16" else 24    # significant bits incl. the hidden one
    return np.where(a > 0, np.ldexp(0.5, e - mant_bits), 0.0)


def compare(g, r, storage, tol=REL_TOL, what=""):
    """Returns a dict of diagnostics; raises AssertionError when parity fails."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in the GPU result"
    diff = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    bound = half_ulp(np.maximum(np.abs(g), np.abs(r)), storage) + tol * np.abs(r) + tol * rms
    ratio = diff / np.where(bound > 0, bound, 1.0)
    worst = float(ratio.max()) if r.size else 0.0
    nr = float(np.linalg.norm(r.ravel()))
    err = float(np.linalg.norm((g - r).ravel()) / nr) if nr > 0 else float(np.linalg.norm(g.ravel()))
    if storage == "bf16" and r.size:
        q = float(np.linalg.norm((si.bf16_bits_to_f64(si.round_bf16_bits(r)) - r).ravel()) / nr) if nr > 0 else 0.0
        excess = float(np.sqrt(max(0.0, err * err - q * q)))
    else:
        q, excess = 0.0, err
    info = dict(what=what, n=int(r.size), max_bound_ratio=worst, normwise=err, storage_q=q,
                excess=excess, max_abs=float(diff.max()) if r.size else 0.0)
    assert worst <= 1.0, f"{what}: elementwise bound exceeded (worst ratio {worst:.3f}); {info}"
    assert excess <= tol, f"{what}: normwise excess {excess:.3e} > {tol}; {info}"
    return info
