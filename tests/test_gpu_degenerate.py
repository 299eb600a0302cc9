"""GPU parity on the degenerate inputs the recurrence admits, against the fp64
oracle on the same stored bits: no decay (A = 0, the state a running sum), identity
steps (Delta = 0: the state passes through unchanged), full decay (Delta A so
negative that exp(Delta A) is zero in fp32: the state is the step's own input term),
decays that underflow, and a zero input with an initial state (pure decay).
Each case spans several segments (and chunks) with a ragged tail, so the carries
between them see the degenerate values too."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ssa
import ssm_inputs as si
from gpu_util import DEV, gpu_scan, gpu_scan_bwd, oracle_scan, oracle_scan_bwd, out_f64, storage
from parity import compare

pytestmark = pytest.mark.gpu

KINDS = ("A0", "A0_half", "dt0_run", "dt0_all", "dt_big", "A_underflow", "x0_h0")


def _degenerate(w, kind, delta_key="delta"):
    """Apply one degenerate pattern to stored inputs (in place); returns w."""
    dt = w["dtype"]
    A = w["A"]
    dl = si.to_f64(w[delta_key])
    L = dl.shape[1]
    if kind == "A0":
        w["A"] = np.zeros_like(A)
    elif kind == "A0_half":  # every other state (scan) or head (SSD) without decay
        A = A.copy()
        A[..., ::2] = 0.0
        w["A"] = A
    elif kind == "dt0_run":  # a run of identity steps across segment and chunk boundaries
        dl = dl.copy()
        dl[:, L // 5: (3 * L) // 5] = 0.0
        w[delta_key] = si.store(dl, dt)
    elif kind == "dt0_all":
        w[delta_key] = si.store(np.zeros_like(dl), dt)
    elif kind == "dt_big":  # exp(40 A) <= e^-40 for A <= -1: nothing survives a step
        w[delta_key] = si.store(np.full_like(dl, 40.0), dt)
    elif kind == "A_underflow":  # exp2 of about -1e4 Delta: zero or subnormal in fp32
        A = A.copy()
        A[..., :2] = -1.0e4
        w["A"] = A
    elif kind == "x0_h0":
        w["x"] = si.store(np.zeros_like(si.to_f64(w["x"])), dt)
    else:
        raise ValueError(kind)
    return w


SCAN_SHAPES = [
    # B, L, D, N, dtype
    (2, 700, 96, 16, si.BF16),
    (1, 1500, 64, 8, si.F32),
    (1, 400, 70, 64, si.BF16),
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", SCAN_SHAPES, ids=lambda c: "B{}_L{}_D{}_N{}_{}".format(*c[:4], c[4]))
def test_scan_degenerate_inputs(shape, kind):
    B, L, D, N, dt = shape
    print(f"[degenerate scan] {shape} {kind}", flush=True)
    w = _degenerate(si.scan_inputs(B, L, D, N, dtype=dt, seed=21, with_h0=True), kind)
    y, hf = gpu_scan(w)
    yr, hr = oracle_scan(w)
    compare(out_f64(y), yr, storage(w), what=f"{kind} y")
    compare(out_f64(hf), hr, "f32", what=f"{kind} h_final")
    if kind == "dt0_all":
        # identity steps: the state is carried through exactly
        np.testing.assert_array_equal(out_f64(hf), w["h0"].astype(np.float64))


SSD_SHAPES = [
    # B, L, H, N, chunk
    (1, 300, 2, 128, 64),
    (2, 257, 3, 64, 256),
]


@pytest.mark.parametrize("kind", [k for k in KINDS if k != "A_underflow"] + ["A_underflow_head"])
@pytest.mark.parametrize("shape", SSD_SHAPES, ids=lambda c: "B{}_L{}_H{}_N{}_Q{}".format(*c))
def test_ssd_degenerate_inputs(shape, kind):
    B, L, H, N, Q = shape
    print(f"[degenerate ssd] {shape} {kind}", flush=True)
    w = si.ssd_inputs(B, L, H, 64, N, dtype=si.BF16, seed=22, with_D=True, with_z=True, with_h0=True)
    if kind == "A_underflow_head":
        A = w["A"].copy()
        A[0] = -1.0e4
        w["A"] = A
    else:
        w = _degenerate(w, kind)
    t = {k: (si.to_torch(w[k], DEV) if w.get(k) is not None else None)
         for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    y, hf = ssa.ssm_ssd_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"], h0=t["h0"],
                            chunk=Q)
    torch.cuda.synchronize()
    f = {k: si.to_f64(w[k]) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    yr, hr = oracle.ssd_seq(f["x"], f["delta"], f["A"], f["Bm"], f["Cm"], D=f["D"], z=f["z"], h0=f["h0"])
    compare(out_f64(y), yr, "bf16", what=f"{kind} y")
    compare(out_f64(hf), hr, "f32", what=f"{kind} h_final")


@pytest.mark.parametrize("kind", ("A0", "dt0_run", "dt0_all", "dt_big", "x0_h0"))
def test_step_degenerate_inputs(kind):
    """Decode steps chained in place; Delta = 0 leaves the state bit for bit."""
    B, D, N, steps = 2, 130, 16, 40
    print(f"[degenerate step] {kind}", flush=True)
    w = si.step_inputs(B, D, N, steps, dtype=si.BF16, seed=23, with_D=True, with_z=True)
    # the per-token arrays are [steps, B, D]: the same patterns along the token axis
    tw = dict(w)
    for k in ("x", "delta"):
        tw[k] = np.ascontiguousarray(np.swapaxes(w[k], 0, 1))
    tw = _degenerate(tw, kind)
    for k in ("x", "delta"):
        w[k] = np.ascontiguousarray(np.swapaxes(tw[k], 0, 1))
    w["A"] = tw["A"]
    st_g = torch.from_numpy(w["state0"]).to(DEV)
    st_o = w["state0"].astype(np.float64)
    A = torch.from_numpy(w["A"]).to(DEV)
    Dk = torch.from_numpy(w["D"]).to(DEV)
    Af, Df = w["A"].astype(np.float64), w["D"].astype(np.float64)
    for s in range(steps):
        tok = {k: w[k][s] for k in ("x", "delta", "z", "Bm", "Cm")}
        td = {k: si.to_torch(np.ascontiguousarray(v), DEV) for k, v in tok.items()}
        y = ssa.ssm_step(st_g, td["x"], td["delta"], A, td["Bm"], td["Cm"], D=Dk, z=td["z"])
        yo, st_o = oracle.step(st_o, si.to_f64(tok["x"]), si.to_f64(tok["delta"]), Af, si.to_f64(tok["Bm"]),
                               si.to_f64(tok["Cm"]), D=Df, z=si.to_f64(tok["z"]))
        torch.cuda.synchronize()
        compare(out_f64(y), yo, "bf16", what=f"{kind} step {s} y")
    compare(st_g.cpu().numpy(), st_o, "f32", what=f"{kind} state")
    if kind == "dt0_all":
        np.testing.assert_array_equal(st_g.cpu().numpy(), w["state0"])


BWD_SHAPES = [
    # B, L, D, N, dtype
    (2, 300, 70, 16, si.BF16),
    (1, 200, 64, 64, si.F32),
    (1, 130, 70, 128, si.BF16),
]


# Under full decay (dt_big) the gradient of A is analytically ~e^-40 of its usual size;
# the kernel forms a_t h_{t-1} from h_{t-1} itself, so it still matches at its own scale.
# Underflow on two states keeps the other states' scale.
@pytest.mark.parametrize("kind", ("A0", "A0_half", "dt0_run", "dt_big", "A_underflow", "x0_h0"))
@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda c: "B{}_L{}_D{}_N{}_{}".format(*c[:4], c[4]))
def test_scan_bwd_degenerate_inputs(shape, kind):
    B, L, D, N, dt = shape
    print(f"[degenerate bwd] {shape} {kind}", flush=True)
    w = _degenerate(si.scan_inputs(B, L, D, N, dtype=dt, seed=24, with_h0=True), kind)
    gw = si.scan_grad_inputs(B, L, D, N, dtype=dt, seed=25)
    g = gpu_scan_bwd(w, gw)
    r = oracle_scan_bwd(w, gw)
    st = storage(w)
    for k in ("dx", "ddelta", "dz", "dBm", "dCm", "dA", "dD", "dh0"):
        compare(out_f64(g[k]), r[k], st if k in ("dx", "ddelta", "dz", "dBm", "dCm") else "f32", what=f"{kind} {k}")


# ---------------------------------------------------------------- the other paths

@pytest.mark.parametrize("kind", ("A0", "dt0_all", "dt_big", "x0"))
def test_ssd_step_degenerate_inputs(kind):
    """Mamba-2 decode chained in place: no decay, identity steps (the state bit for
    bit), full decay, zero input."""
    B, H, N, steps = 2, 3, 128, 20
    print(f"[degenerate ssd step] {kind}", flush=True)
    w = si.ssd_step_inputs(B, H, 64, N, steps, dtype=si.BF16, seed=26, with_D=True, with_z=True)
    dl = si.to_f64(w["delta"])
    if kind == "A0":
        w["A"] = np.zeros_like(w["A"])
    elif kind == "dt0_all":
        w["delta"] = si.store(np.zeros_like(dl), si.BF16)
    elif kind == "dt_big":
        w["delta"] = si.store(np.full_like(dl, 40.0), si.BF16)
    else:
        w["x"] = si.store(np.zeros_like(si.to_f64(w["x"])), si.BF16)
    st_g = torch.from_numpy(w["state0"]).to(DEV)
    st_o = w["state0"].astype(np.float64)
    A, Dk = torch.from_numpy(w["A"]).to(DEV), torch.from_numpy(w["D"]).to(DEV)
    for s in range(steps):
        tok = {k: w[k][s] for k in ("x", "delta", "z", "Bm", "Cm")}
        td = {k: si.to_torch(np.ascontiguousarray(v), DEV) for k, v in tok.items()}
        y = ssa.ssm_ssd_step(st_g, td["x"], td["delta"], A, td["Bm"], td["Cm"], D=Dk, z=td["z"])
        yo, st_o = oracle.ssd_step(st_o, si.to_f64(tok["x"]), si.to_f64(tok["delta"]), w["A"].astype(np.float64),
                                   si.to_f64(tok["Bm"]), si.to_f64(tok["Cm"]), D=w["D"].astype(np.float64),
                                   z=si.to_f64(tok["z"]))
        torch.cuda.synchronize()
        compare(out_f64(y), yo, "bf16", what=f"{kind} step {s} y")
    compare(st_g.cpu().numpy(), st_o, "f32", what=f"{kind} state")
    if kind == "dt0_all":
        np.testing.assert_array_equal(st_g.cpu().numpy(), w["state0"])


@pytest.mark.parametrize("case", [
    # kind, disc, softplus, N
    ("dt_big", "zoh", False, 16), ("dt_big", "zoh", False, 64), ("dt0_run", "zoh", False, 16),
    ("A0", "zoh", False, 16), ("raw_pos", "zoh", True, 16), ("raw_neg", "zoh", True, 64),
    ("raw_pos", "euler", True, 16), ("raw_neg", "euler", True, 16),
], ids=lambda c: "{}_{}_sp{}_N{}".format(*c))
def test_scan_variant_degenerate_inputs(case):
    """The discretisation variants at the extremes: zero-order hold under full decay
    (e^z - 1 -> -1), identity steps and A = 0 (its limit Delta), and softplus(delta +
    bias) of raw values around +-80 (Delta ~ 75, or ~ e^-85 where only the series holds)."""
    from test_gpu_scan_var import _run
    kind, disc, sp, N = case
    print(f"[degenerate variant] {case}", flush=True)
    B, L, D = 2, 300, 70
    w = si.scan_inputs(B, L, D, N, dtype=si.BF16, seed=27, with_h0=True)
    bias = None
    if kind in ("raw_pos", "raw_neg"):
        r = si.scan_raw_delta(B, L, D, dtype=si.BF16, seed=27)
        raw = si.to_f64(r["delta"])
        raw[:, L // 4: L // 2] = 80.0 if kind == "raw_pos" else -80.0
        w["delta"], bias = si.store(raw, si.BF16), r["delta_bias"]
    else:
        w = _degenerate(w, kind)
    (y, hf), (yr, hr) = _run(w, bias, disc, sp)
    compare(out_f64(y), yr, "bf16", what=f"{case} y")
    compare(out_f64(hf), hr, "f32", what=f"{case} h_final")


def _mamba3_degenerate(w, kind):
    dl = si.to_f64(w["delta"])
    L = dl.shape[1]
    if kind == "theta_big":  # up to tens of radians per step, many turns per segment
        w["theta"] = np.random.default_rng(28).uniform(-200.0, 200.0, w["theta"].shape).astype(np.float32)
    elif kind == "Are0":     # |alpha| = 1: rotation only
        w["Are"] = np.zeros_like(w["Are"])
    elif kind in ("lam0", "lam1"):
        w["lam"] = si.store(np.full_like(si.to_f64(w["lam"]), 0.0 if kind == "lam0" else 1.0), w["dtype"])
    elif kind == "dt0_run":
        dl = dl.copy()
        dl[:, L // 5: (3 * L) // 5] = 0.0
        w["delta"] = si.store(dl, w["dtype"])
    elif kind == "dt_big":
        w["delta"] = si.store(np.full_like(dl, 40.0), w["dtype"])
    else:
        raise ValueError(kind)
    return w


@pytest.mark.parametrize("kind", ("theta_big", "Are0", "lam0", "lam1", "dt0_run", "dt_big"))
def test_scan3_degenerate_inputs(kind):
    """Mamba-3 scan: phases of many turns, no magnitude decay, the two ends of the
    trapezoid weight, identity steps and full decay, across segments with a ragged tail."""
    from test_gpu_scan3 import gpu_scan3, oracle_scan3
    print(f"[degenerate scan3] {kind}", flush=True)
    w = _mamba3_degenerate(si.scan3_inputs(2, 700, 96, 16, dtype=si.BF16, seed=28, with_h0=True, with_prev=True),
                           kind)
    y, hf = gpu_scan3(w)
    yr, hr = oracle_scan3(w)
    compare(out_f64(y), yr, "bf16", what=f"{kind} y")
    compare(out_f64(hf), hr, "f32", what=f"{kind} h_final")


@pytest.mark.parametrize("kind", ("theta_big", "Are0", "lam0", "dt_big"))
def test_step3_degenerate_inputs(kind):
    """Mamba-3 decode chained over 30 tokens against the oracle's scan over them."""
    from test_gpu_scan3 import oracle_scan3
    from test_gpu_step3 import _start, gpu_steps
    print(f"[degenerate step3] {kind}", flush=True)
    w = _mamba3_degenerate(si.scan3_inputs(2, 30, 70, 16, dtype=si.BF16, seed=29, with_h0=True, with_prev=True),
                           kind)
    st, prev = _start(w)
    y = gpu_steps(w, 0, 30, st, prev)
    yr, hr = oracle_scan3(w)
    compare(out_f64(y), yr, "bf16", what=f"{kind} y")
    compare(st.cpu().numpy().astype(np.float64), hr, "f32", what=f"{kind} state")
