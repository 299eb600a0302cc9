"""GPU parity of ssm_scan3_fwd (Mamba-3: complex transitions, exponential-trapezoidal
rule) against the fp64 oracle O8."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ssa
import ssm_inputs as si
from gpu_util import DEV, out_f64, storage
from parity import compare

pytestmark = pytest.mark.gpu

KEYS = ("x", "delta", "lam", "Are", "theta", "Bm", "Cm", "D", "z", "h0", "x_prev", "B_prev")


def gpu_scan3(w, **kw):
    t = {k: (si.to_torch(w[k], DEV) if w.get(k) is not None else None) for k in KEYS}
    y, hf = ssa.ssm_scan3_fwd(t["x"], t["delta"], t["lam"], t["Are"], t["theta"], t["Bm"], t["Cm"], D=t["D"],
                              z=t["z"], h0=t["h0"], x_prev=t["x_prev"], B_prev=t["B_prev"], **kw)
    torch.cuda.synchronize()
    return y, hf


def oracle_scan3(w):
    f = {k: (si.to_f64(w[k]) if w.get(k) is not None else None) for k in KEYS}
    h0 = None if f["h0"] is None else f["h0"][..., 0] + 1j * f["h0"][..., 1]
    y, hf = oracle.scan3(f["x"], f["delta"], f["lam"], f["Are"], f["theta"], f["Bm"], f["Cm"], D=f["D"], z=f["z"],
                         h0=h0, x_prev=f["x_prev"], B_prev=f["B_prev"])
    return y, np.stack([hf.real, hf.imag], axis=-1)


def _check(w, what):
    y, hf = gpu_scan3(w)
    yr, hr = oracle_scan3(w)
    compare(out_f64(y), yr, storage(w), what=f"{what} y")
    compare(out_f64(hf), hr, "f32", what=f"{what} h_final")


SMALL = [
    # B, L, D, N, dtype, with_D, with_z, with_h0, with_prev
    (1, 1, 64, 16, si.F32, True, True, True, True),
    (2, 37, 70, 16, si.BF16, True, True, True, False),
    (1, 300, 64, 4, si.F32, False, False, False, False),
    (3, 1000, 130, 8, si.BF16, True, False, True, True),
    (1, 2000, 96, 16, si.F32, True, True, False, True),
    (2, 4097, 200, 16, si.BF16, True, True, True, True),
    (5, 77, 1, 8, si.F32, True, True, True, False),
    # one group of two to four segments runs as one launch
    (3, 100, 130, 16, si.BF16, True, True, True, True),
    (16, 128, 1024, 16, si.BF16, True, True, False, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_L{}_D{}_N{}_{}_D{}z{}h{}p{}".format(*c))
def test_scan3_small_shapes(case):
    B, L, D, N, dt, wd, wz, wh, wp = case
    print(f"[scan3 small] {case}", flush=True)
    w = si.scan3_inputs(B, L, D, N, dtype=dt, seed=51, with_D=wd, with_z=wz, with_h0=wh, with_prev=wp)
    _check(w, str(case))


def test_scan3_workload_bf16_B1_L4096_D1536_N16():
    print("[scan3] bf16 B1 L4096 D1536 N16 (every element)", flush=True)
    w = si.scan3_inputs(1, 4096, 1536, 16, dtype=si.BF16, seed=0)
    _check(w, "scan3 layer")


def test_scan3_euler_limit_matches_scan():
    """lam = 1, theta = 0: the Mamba-3 kernels give the Mamba-1 scan's result."""
    w = si.scan3_inputs(2, 3000, 128, 16, dtype=si.F32, seed=52, with_h0=True)
    w["lam"] = np.ones_like(w["lam"])
    w["theta"] = np.zeros_like(w["theta"])
    w["h0"][..., 1] = 0.0
    y3, h3 = gpu_scan3(w)
    t = {k: si.to_torch(w[k], DEV) for k in ("x", "delta", "Bm", "Cm", "D", "z")}
    y1, h1 = ssa.ssm_scan_fwd(t["x"], t["delta"], si.to_torch(w["Are"], DEV), t["Bm"], t["Cm"], D=t["D"], z=t["z"],
                              h0=si.to_torch(np.ascontiguousarray(w["h0"][..., 0]), DEV))
    torch.cuda.synchronize()
    compare(out_f64(y3), out_f64(y1), "f32", tol=1e-5, what="euler limit y")
    compare(out_f64(h3)[..., 0], out_f64(h1), "f32", tol=1e-5, what="euler limit h")
    assert np.max(np.abs(out_f64(h3)[..., 1])) == 0.0


def test_scan3_split_carry_on_gpu():
    """scan3(x[:m]) then scan3(x[m:]) from its final state and last token == scan3(x)."""
    w = si.scan3_inputs(2, 3000, 96, 16, dtype=si.F32, seed=53, with_h0=True, with_prev=True)
    y, hf = gpu_scan3(w)
    m = 1234
    seq = ("x", "delta", "lam", "z", "Bm", "Cm")
    w1 = dict(w, **{k: np.ascontiguousarray(w[k][:, :m]) for k in seq})
    y1, h1 = gpu_scan3(w1)
    w2 = dict(w, **{k: np.ascontiguousarray(w[k][:, m:]) for k in seq})
    w2.update(h0=h1.cpu().numpy(), x_prev=np.ascontiguousarray(w["x"][:, m - 1]),
              B_prev=np.ascontiguousarray(w["Bm"][:, m - 1]))
    y2, h2 = gpu_scan3(w2)
    compare(np.concatenate([out_f64(y1), out_f64(y2)], axis=1), out_f64(y), "f32", what="split y")
    compare(out_f64(h2), out_f64(hf), "f32", what="split h")


def test_scan3_empty_sequence_returns_initial_state():
    w = si.scan3_inputs(2, 0, 64, 8, dtype=si.BF16, seed=54, with_h0=True)
    y, hf = gpu_scan3(w)
    assert y.shape == (2, 0, 64)
    np.testing.assert_array_equal(out_f64(hf), w["h0"].astype(np.float64))
