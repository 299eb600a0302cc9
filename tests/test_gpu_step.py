"""GPU parity of ssm_step (recurrent decode) against the fp64 oracle, and the
step == prefill relations on the GPU."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ssa
import ssm_inputs as si
from gpu_util import DEV, gpu_scan, out_f64, storage
from parity import compare

pytestmark = pytest.mark.gpu


def _run_steps(w, steps):
    """Chain `steps` GPU decode steps and the same oracle steps; compare every y and the state."""
    st_g = torch.from_numpy(w["state0"]).to(DEV)
    st_o = w["state0"].astype(np.float64)
    A = torch.from_numpy(w["A"]).to(DEV)
    Dk = None if w["D"] is None else torch.from_numpy(w["D"]).to(DEV)
    Af, Df = w["A"].astype(np.float64), None if w["D"] is None else w["D"].astype(np.float64)
    for s in range(steps):
        tok = {k: (None if w[k] is None else w[k][s]) for k in ("x", "delta", "z", "Bm", "Cm")}
        td = {k: (None if v is None else si.to_torch(np.ascontiguousarray(v), DEV)) for k, v in tok.items()}
        y = ssa.ssm_step(st_g, td["x"], td["delta"], A, td["Bm"], td["Cm"], D=Dk, z=td["z"])
        yo, st_o = oracle.step(st_o, si.to_f64(tok["x"]), si.to_f64(tok["delta"]), Af,
                               si.to_f64(tok["Bm"]), si.to_f64(tok["Cm"]), D=Df, z=si.to_f64(tok["z"]))
        torch.cuda.synchronize()
        compare(out_f64(y), yo, storage(w), what=f"step {s} y")
    compare(st_g.cpu().numpy(), st_o, "f32", what="state after steps")


@pytest.mark.parametrize("case", [
    (1, 64, 16, si.BF16, True, True), (3, 100, 4, si.F32, False, False),
    (2, 1000, 8, si.BF16, True, False), (4, 300, 32, si.F32, False, True),
    (2, 130, 64, si.BF16, True, True), (1, 1, 16, si.F32, True, True),
    (2, 70, 128, si.BF16, True, True), (3, 33, 256, si.F32, False, True),
], ids=lambda c: "B{}_D{}_N{}_{}_D{}z{}".format(*c))
def test_step_small(case):
    B, D, N, dt, wd, wz = case
    print(f"[step small] {case}", flush=True)
    w = si.step_inputs(B, D, N, steps=12, dtype=dt, seed=3, with_D=wd, with_z=wz)
    _run_steps(w, 12)


def test_step_config_bf16_B64_D3072_N16_1000_steps():
    """The decode workload as stated: 1000 consecutive in-place steps on the GPU
    (queued back to back, no synchronisation between them), then the same chain on
    the oracle; y compared at every step, the state after every 100th step."""
    steps, every = 1000, 100
    print(f"[step] bf16 B64 D3072 N16, {steps} chained in-place steps", flush=True)
    w = si.step_inputs(64, 3072, 16, steps=steps, dtype=si.BF16, seed=0)
    tok = {k: si.to_torch(w[k], DEV) for k in ("x", "delta", "z", "Bm", "Cm")}
    A = torch.from_numpy(w["A"]).to(DEV)
    Dk = torch.from_numpy(w["D"]).to(DEV)
    st = torch.from_numpy(w["state0"]).to(DEV)
    y = torch.empty((steps, 64, 3072), dtype=torch.bfloat16, device=DEV)
    snaps = []
    for s in range(steps):
        ssa.ssm_step(st, tok["x"][s], tok["delta"][s], A, tok["Bm"][s], tok["Cm"][s], D=Dk, z=tok["z"][s],
                     y=y[s])
        if (s + 1) % every == 0:
            snaps.append(st.clone())
    torch.cuda.synchronize()
    yg = out_f64(y)
    sg = [t.cpu().numpy().astype(np.float64) for t in snaps]
    st_o = w["state0"].astype(np.float64)
    Af, Df = w["A"].astype(np.float64), w["D"].astype(np.float64)
    for s in range(steps):
        yo, st_o = oracle.step(st_o, si.to_f64(w["x"][s]), si.to_f64(w["delta"][s]), Af, si.to_f64(w["Bm"][s]),
                               si.to_f64(w["Cm"][s]), D=Df, z=si.to_f64(w["z"][s]))
        compare(yg[s], yo, "bf16", what=f"step {s} y")
        if (s + 1) % every == 0:
            info = compare(sg[(s + 1) // every - 1], st_o, "f32", what=f"state after step {s + 1}")
            print(f"  state after {s + 1} steps: normwise {info['normwise']:.2e}", flush=True)


def test_step_equals_prefill_of_one_on_gpu():
    w = si.scan_inputs(2, 1, 320, 16, dtype=si.BF16, seed=8, with_h0=True)
    y, hf = gpu_scan(w)
    st = torch.from_numpy(w["h0"]).to(DEV)
    t = {k: si.to_torch(np.ascontiguousarray(w[k][:, 0]), DEV) for k in ("x", "delta", "z", "Bm", "Cm")}
    ys = ssa.ssm_step(st, t["x"], t["delta"], torch.from_numpy(w["A"]).to(DEV), t["Bm"], t["Cm"],
                      D=torch.from_numpy(w["D"]).to(DEV), z=t["z"])
    torch.cuda.synchronize()
    compare(out_f64(ys), out_f64(y)[:, 0], "bf16", what="step vs L=1 y")
    compare(st.cpu().numpy(), out_f64(hf), "f32", what="step vs L=1 state")


@pytest.mark.parametrize("N", [16, 256])
def test_prefill_then_step_equals_longer_prefill_on_gpu(N):
    L = 777
    w = si.scan_inputs(2, L + 1, 256, N, dtype=si.BF16, seed=9, with_h0=True)
    yfull, hfull = gpu_scan(w)
    cut = {k: np.ascontiguousarray(w[k][:, :L]) for k in ("x", "delta", "z", "Bm", "Cm")}
    _, h = gpu_scan(dict(w, **cut))
    t = {k: si.to_torch(np.ascontiguousarray(w[k][:, L]), DEV) for k in ("x", "delta", "z", "Bm", "Cm")}
    ys = ssa.ssm_step(h, t["x"], t["delta"], torch.from_numpy(w["A"]).to(DEV), t["Bm"], t["Cm"],
                      D=torch.from_numpy(w["D"]).to(DEV), z=t["z"])
    torch.cuda.synchronize()
    compare(out_f64(ys), out_f64(yfull)[:, L], "bf16", what="prefill+step y")
    compare(h.cpu().numpy(), out_f64(hfull), "f32", what="prefill+step state")


def test_step_hip_graph_replay_matches_eager():
    """Ten decode steps captured in a HIP graph and replayed three times, with
    eager work and synchronisations between replays: every replay equals the
    eager result bit for bit."""
    B, D, N, S = 8, 512, 16, 10
    w = si.step_inputs(B, D, N, steps=S, dtype=si.BF16, seed=12)
    tok = {k: si.to_torch(w[k], DEV) for k in ("x", "delta", "z", "Bm", "Cm")}
    A = torch.from_numpy(w["A"]).to(DEV)
    Dk = torch.from_numpy(w["D"]).to(DEV)
    st0 = torch.from_numpy(w["state0"]).to(DEV)

    def run(st, y):
        for s in range(S):
            ssa.ssm_step(st, tok["x"][s], tok["delta"][s], A, tok["Bm"][s], tok["Cm"][s], D=Dk,
                         z=tok["z"][s], y=y[s])

    st_e = st0.clone()
    y_e = torch.empty((S, B, D), dtype=torch.bfloat16, device=DEV)
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
        # unrelated eager work between replays
        _ = (st0 * 2.0).sum().item()
