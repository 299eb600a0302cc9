"""GPU parity of ssm_ssd_step (Mamba-2 recurrent decode) against the fp64 oracle,
and the step == prefill relations against ssm_ssd_fwd on the GPU."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ssa
import ssm_inputs as si
from gpu_util import DEV, out_f64, storage
from parity import compare

pytestmark = pytest.mark.gpu


def _run_steps(w, steps):
    """Chain `steps` GPU steps and the same oracle steps; compare every y and the state."""
    st_g = torch.from_numpy(w["state0"]).to(DEV)
    st_o = w["state0"].astype(np.float64)
    A = torch.from_numpy(w["A"]).to(DEV)
    Dk = None if w["D"] is None else torch.from_numpy(w["D"]).to(DEV)
    Af, Df = w["A"].astype(np.float64), None if w["D"] is None else w["D"].astype(np.float64)
    for s in range(steps):
        tok = {k: (None if w[k] is None else w[k][s]) for k in ("x", "delta", "z", "Bm", "Cm")}
        td = {k: (None if v is None else si.to_torch(np.ascontiguousarray(v), DEV)) for k, v in tok.items()}
        y = ssa.ssm_ssd_step(st_g, td["x"], td["delta"], A, td["Bm"], td["Cm"], D=Dk, z=td["z"])
        yo, st_o = oracle.ssd_step(st_o, si.to_f64(tok["x"]), si.to_f64(tok["delta"]), Af,
                                   si.to_f64(tok["Bm"]), si.to_f64(tok["Cm"]), D=Df, z=si.to_f64(tok["z"]))
        torch.cuda.synchronize()
        compare(out_f64(y), yo, storage(w), what=f"ssd step {s} y")
    compare(st_g.cpu().numpy(), st_o, "f32", what="ssd state after steps")


@pytest.mark.parametrize("case", [
    (1, 1, 64, si.BF16, True, True), (2, 3, 128, si.F32, False, False),
    (3, 2, 16, si.BF16, True, False), (1, 4, 256, si.F32, False, True),
    (2, 5, 32, si.BF16, True, True),
], ids=lambda c: "B{}_H{}_N{}_{}_D{}z{}".format(*c))
def test_ssd_step_small(case):
    B, H, N, dt, wd, wz = case
    print(f"[ssd step small] {case}", flush=True)
    w = si.ssd_step_inputs(B, H, 64, N, steps=12, dtype=dt, seed=4, with_D=wd, with_z=wz)
    _run_steps(w, 12)


def test_ssd_step_config_bf16_B64_H24_P64_N128():
    print("[ssd step] bf16 B64 H24 P64 N128, 10 chained steps", flush=True)
    w = si.ssd_step_inputs(64, 24, 64, 128, steps=10, dtype=si.BF16, seed=0)
    _run_steps(w, 10)


def _ssd_fwd(w, L, h0):
    t = {k: si.to_torch(np.ascontiguousarray(w[k][:, :L]), DEV) for k in ("x", "delta", "z", "Bm", "Cm")}
    return ssa.ssm_ssd_fwd(t["x"], t["delta"], torch.from_numpy(w["A"]).to(DEV), t["Bm"], t["Cm"],
                           D=torch.from_numpy(w["D"]).to(DEV), z=t["z"], h0=h0)


def _step(w, t_idx, st):
    t = {k: si.to_torch(np.ascontiguousarray(w[k][:, t_idx]), DEV) for k in ("x", "delta", "z", "Bm", "Cm")}
    return ssa.ssm_ssd_step(st, t["x"], t["delta"], torch.from_numpy(w["A"]).to(DEV), t["Bm"], t["Cm"],
                            D=torch.from_numpy(w["D"]).to(DEV), z=t["z"])


def test_ssd_step_equals_prefill_of_one_on_gpu():
    w = si.ssd_inputs(2, 1, 3, 64, 128, dtype=si.BF16, seed=10, with_D=True, with_z=True, with_h0=True)
    y, hf = _ssd_fwd(w, 1, torch.from_numpy(w["h0"]).to(DEV))
    st = torch.from_numpy(w["h0"]).to(DEV)
    ys = _step(w, 0, st)
    torch.cuda.synchronize()
    compare(out_f64(ys), out_f64(y)[:, 0], "bf16", what="ssd step vs L=1 y")
    compare(st.cpu().numpy(), out_f64(hf), "f32", what="ssd step vs L=1 state")


def test_ssd_prefill_then_step_equals_longer_prefill_on_gpu():
    L = 300
    w = si.ssd_inputs(2, L + 1, 3, 64, 64, dtype=si.BF16, seed=11, with_D=True, with_z=True, with_h0=True)
    h0 = torch.from_numpy(w["h0"]).to(DEV)
    yfull, hfull = _ssd_fwd(w, L + 1, h0)
    _, h = _ssd_fwd(w, L, h0)
    ys = _step(w, L, h)
    torch.cuda.synchronize()
    compare(out_f64(ys), out_f64(yfull)[:, L], "bf16", what="ssd prefill+step y")
    compare(h.cpu().numpy(), out_f64(hfull), "f32", what="ssd prefill+step state")


def test_ssd_step_hip_graph_replay_matches_eager():
    """Eight steps captured in a HIP graph and replayed three times, with eager
    work and synchronisations between replays: every replay equals the eager
    result bit for bit."""
    B, H, N, S = 4, 6, 128, 8
    w = si.ssd_step_inputs(B, H, 64, N, steps=S, dtype=si.BF16, seed=13)
    tok = {k: si.to_torch(w[k], DEV) for k in ("x", "delta", "z", "Bm", "Cm")}
    A = torch.from_numpy(w["A"]).to(DEV)
    Dk = torch.from_numpy(w["D"]).to(DEV)
    st0 = torch.from_numpy(w["state0"]).to(DEV)

    def run(st, y):
        for s in range(S):
            ssa.ssm_ssd_step(st, tok["x"][s], tok["delta"][s], A, tok["Bm"][s], tok["Cm"][s], D=Dk,
                             z=tok["z"][s], y=y[s])

    st_e = st0.clone()
    y_e = torch.empty((S, B, H, 64), dtype=torch.bfloat16, device=DEV)
    run(st_e, y_e)
    torch.cuda.synchronize()
    st_g = st0.clone()
    y_g = torch.empty_like(y_e)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run(st_g, y_g)
    torch.cuda.synchronize()
    for rep in range(3):
        st_g.copy_(st0)
        y_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {rep}: y differs from eager"
        assert torch.equal(st_g, st_e), f"replay {rep}: state differs from eager"
        _ = (st0 * 2.0).sum().item()
