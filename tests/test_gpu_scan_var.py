"""GPU parity of the discretisation variants (ssm_scan_fwd_ex, ssm_step_ex):
exact zero-order hold and Delta = softplus(delta + bias) in the kernels, against
the fp64 oracle's O7 on the same stored inputs."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ssa
import ssm_inputs as si
from gpu_util import DEV, out_f64, storage
from parity import compare

pytestmark = pytest.mark.gpu


def _inputs(B, L, D, N, dt, seed, raw, with_D, with_z, with_h0, A=None, delta_scale=None, softplus=True):
    """raw: a delta_bias is passed; with softplus, Delta is drawn before its softplus
    (the workload's own distribution after it); without, Delta stays positive and
    the bias is a small positive shift (a step must stay positive)."""
    w = si.scan_inputs(B, L, D, N, dtype=dt, seed=seed, with_D=with_D, with_z=with_z, with_h0=with_h0)
    bias = None
    if raw and softplus:
        r = si.scan_raw_delta(B, L, D, dtype=dt, seed=seed)
        w["delta"], bias = r["delta"], r["delta_bias"]
    elif raw:
        bias = (0.01 * np.abs(np.random.default_rng(seed).standard_normal(D))).astype(np.float32)
    if delta_scale is not None:  # tiny Delta: every |z| small
        w["delta"] = si.store(si.to_f64(w["delta"]) * delta_scale, dt)
    if A is not None:
        w["A"] = np.ascontiguousarray(A, dtype=np.float32)
    return w, bias


def _run(w, bias, disc, sp):
    t = {k: (si.to_torch(w[k], DEV) if w.get(k) is not None else None)
         for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    bt = None if bias is None else torch.from_numpy(bias).to(DEV)
    y, hf = ssa.ssm_scan_fwd_ex(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"], h0=t["h0"],
                                disc=disc, delta_bias=bt, delta_softplus=sp)
    torch.cuda.synchronize()
    f = {k: si.to_f64(w[k]) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    yr, hr = oracle.scan_disc(f["x"], f["delta"], f["A"], f["Bm"], f["Cm"], D=f["D"], z=f["z"], h0=f["h0"],
                              disc=disc, delta_bias=None if bias is None else bias.astype(np.float64),
                              delta_softplus=sp)
    return (y, hf), (yr, hr)


CASES = [
    # B, L, D, N, dtype, disc, raw delta + bias, softplus, with_D, with_z, with_h0
    (1, 1, 64, 16, si.F32, "zoh", False, False, True, True, True),
    (2, 37, 70, 16, si.BF16, "zoh", True, True, True, True, True),
    (1, 300, 64, 4, si.F32, "zoh", False, False, False, False, False),
    (3, 1000, 130, 8, si.BF16, "euler", True, True, True, False, True),
    (1, 2000, 32, 32, si.F32, "zoh", True, True, True, True, False),
    (2, 513, 200, 16, si.BF16, "euler", True, False, True, True, True),
    (1, 4097, 96, 16, si.BF16, "zoh", True, True, False, True, False),
    (5, 77, 1, 16, si.F32, "zoh", True, True, True, True, True),
    # N >= 64: chunks of 16 states, partial sums added across the chunks
    (2, 300, 70, 64, si.BF16, "zoh", True, True, True, True, True),
    (1, 1000, 96, 128, si.F32, "euler", True, True, False, True, False),
    (1, 257, 64, 256, si.BF16, "zoh", True, True, True, False, True),
    (3, 129, 130, 64, si.F32, "euler", True, False, False, False, True),
    # short chains in one launch
    (2, 100, 70, 16, si.BF16, "zoh", True, True, True, True, True),
    (32, 256, 1024, 16, si.BF16, "zoh", True, True, True, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_L{}_D{}_N{}_{}_{}_raw{}_sp{}_D{}z{}h{}".format(*c))
def test_scan_variant_small_shapes(case):
    B, L, D, N, dt, disc, raw, sp, wd, wz, wh = case
    print(f"[scan_var] {case}", flush=True)
    w, bias = _inputs(B, L, D, N, dt, 11, raw, wd, wz, wh, softplus=sp)
    (y, hf), (yr, hr) = _run(w, bias, disc, sp)
    compare(out_f64(y), yr, storage(w), what=f"{case} y")
    compare(out_f64(hf), hr, "f32", what=f"{case} h_final")


@pytest.mark.parametrize("N", [16, 64])
@pytest.mark.parametrize("scale", [1e-3, 0.05])
def test_scan_zoh_small_z_and_zero_A(scale, N):
    """Tiny Delta (every |z| below the switch: the blended series path) and mixed
    scales, with A holding exact zeros and a positive entry."""
    B, L, D = 2, 700, 96
    A = -np.tile(np.arange(1, N + 1, dtype=np.float64), (D, 1))
    A[:, 0] = 0.0
    A[::7, 5] = 0.25
    A[::5, N - 3] = 0.0
    w, _ = _inputs(B, L, D, N, si.F32, 12, False, True, True, True, A=A, delta_scale=scale)
    (y, hf), (yr, hr) = _run(w, None, "zoh", False)
    compare(out_f64(y), yr, "f32", what=f"zoh scale {scale} N{N} y")
    compare(out_f64(hf), hr, "f32", what=f"zoh scale {scale} N{N} h_final")


def test_scan_zoh_softplus_headline_layer():
    """B=1, L=4096, D=1536, N=16, bf16: Delta drawn through the fused softplus(delta + bias)
    (the workload's own distribution), exact zero-order hold; every output."""
    print("[scan_var] zoh softplus B1 L4096 D1536 N16", flush=True)
    w, bias = _inputs(1, 4096, 1536, 16, si.BF16, 0, True, True, True, False)
    (y, hf), (yr, hr) = _run(w, bias, "zoh", True)
    compare(out_f64(y), yr, "bf16", what="headline zoh y")
    compare(out_f64(hf), hr, "f32", what="headline zoh h_final")


@pytest.mark.parametrize("N", [64, 128, 256])
def test_scan_zoh_softplus_state_dim_sweep(N):
    """The state-dimension sweep shape B=1, L=4096, D=1536, N = 64 / 128 / 256, bf16,
    with Delta through the fused softplus(delta + bias) and exact zero-order hold;
    every output."""
    print(f"[scan_var] zoh softplus B1 L4096 D1536 N{N}", flush=True)
    w, bias = _inputs(1, 4096, 1536, N, si.BF16, 1, True, True, True, False)
    (y, hf), (yr, hr) = _run(w, bias, "zoh", True)
    compare(out_f64(y), yr, "bf16", what=f"sweep N{N} zoh y")
    compare(out_f64(hf), hr, "f32", what=f"sweep N{N} zoh h_final")


@pytest.mark.parametrize("disc", ["euler", "zoh"])
def test_prefill_ex_then_steps_ex(disc):
    """prefill(L) with ssm_scan_fwd_ex, then tokens with ssm_step_ex, equals the oracle
    walking the same options; also ssm_step_ex alone at N = 64 (all N are supported)."""
    B, L, D, N, S = 2, 300, 128, 16, 4
    w, bias = _inputs(B, L + S, D, N, si.BF16, 13, True, True, True, True)
    pre = {k: (np.ascontiguousarray(v[:, :L]) if k in ("x", "delta", "z", "Bm", "Cm") else v) for k, v in w.items()}
    (y, hf), (yr, hr) = _run(pre, bias, disc, True)
    compare(out_f64(hf), hr, "f32", what=f"{disc} prefill h")
    st = hf.clone()
    so = hr.copy()
    bt = torch.from_numpy(bias).to(DEV)
    Ad, Dd = torch.from_numpy(w["A"]).to(DEV), torch.from_numpy(w["D"]).to(DEV)
    for k in range(S):
        tok = {n: np.ascontiguousarray(w[n][:, L + k]) for n in ("x", "delta", "z", "Bm", "Cm")}
        tt = {n: si.to_torch(tok[n], DEV) for n in tok}
        yk = ssa.ssm_step_ex(st, tt["x"], tt["delta"], Ad, tt["Bm"], tt["Cm"], D=Dd, z=tt["z"], disc=disc,
                             delta_bias=bt, delta_softplus=True)
        yo, so = oracle.step_disc(so, *(si.to_f64(tok[n]) for n in ("x", "delta")), w["A"].astype(np.float64),
                                  si.to_f64(tok["Bm"]), si.to_f64(tok["Cm"]), D=w["D"].astype(np.float64),
                                  z=si.to_f64(tok["z"]), disc=disc, delta_bias=bias.astype(np.float64),
                                  delta_softplus=True)
        torch.cuda.synchronize()
        compare(out_f64(yk), yo, "bf16", what=f"{disc} step {k} y")
    compare(out_f64(st), so, "f32", what=f"{disc} steps state")
    # N = 64 decode with the options (the variant step covers every N)
    s64 = si.step_inputs(3, 256, 64, steps=1, dtype=si.F32, seed=14)
    b64 = np.linspace(-1.0, 0.5, 256).astype(np.float32)
    st64 = torch.from_numpy(s64["state0"]).to(DEV)
    tok = {n: si.to_torch(np.ascontiguousarray(s64[n][0]), DEV) for n in ("x", "delta", "z", "Bm", "Cm")}
    y64 = ssa.ssm_step_ex(st64, tok["x"], tok["delta"], torch.from_numpy(s64["A"]).to(DEV), tok["Bm"], tok["Cm"],
                          D=torch.from_numpy(s64["D"]).to(DEV), z=tok["z"], disc=disc,
                          delta_bias=torch.from_numpy(b64).to(DEV), delta_softplus=True)
    yo, so = oracle.step_disc(s64["state0"].astype(np.float64), *(si.to_f64(s64[n][0]) for n in ("x", "delta")),
                              s64["A"].astype(np.float64), si.to_f64(s64["Bm"][0]), si.to_f64(s64["Cm"][0]),
                              D=s64["D"].astype(np.float64), z=si.to_f64(s64["z"][0]), disc=disc,
                              delta_bias=b64.astype(np.float64), delta_softplus=True)
    torch.cuda.synchronize()
    compare(out_f64(y64), yo, "f32", what=f"{disc} N64 step y")
    compare(out_f64(st64), so, "f32", what=f"{disc} N64 step state")


def test_ex_with_plain_options_is_plain_scan():
    """disc = euler with no bias and no softplus takes the plain path: bit-identical."""
    w = si.scan_inputs(2, 900, 128, 16, dtype=si.BF16, seed=15, with_h0=True)
    t = {k: (si.to_torch(w[k], DEV) if w.get(k) is not None else None)
         for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    y1, h1 = ssa.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"], h0=t["h0"])
    y2, h2 = ssa.ssm_scan_fwd_ex(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"], h0=t["h0"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
