"""GPU parity of ssm_step3 (the Mamba-3 one-token decode step, complex state in
place) against the fp64 oracle O8: a run of steps from a state, each given the
previous token, is the Mamba-3 scan over those tokens from that state."""
import numpy as np
import pytest
import torch

import selective_scan_amd as ssa
import ssm_inputs as si
from gpu_util import DEV, out_f64, storage
from parity import compare
from test_gpu_scan3 import gpu_scan3, oracle_scan3

pytestmark = pytest.mark.gpu

SEQ = ("x", "delta", "lam", "Bm", "Cm", "z")


def _dev(w):
    return {k: (si.to_torch(v, DEV) if v is not None else None) for k, v in w.items()
            if v is None or isinstance(v, np.ndarray)}


def gpu_steps(w, t0, t1, state, prev, graph_check=False):
    """ssm_step3 over tokens t0 .. t1-1 of the sequence inputs w, from `state` (a
    device tensor, updated in place); prev = (x_prev, B_prev) device tensors or None.
    Returns the outputs [B, t1 - t0, D] as a device tensor."""
    t = _dev(w)
    ys = []
    for s in range(t0, t1):
        tok = {k: (t[k][:, s].clone() if t.get(k) is not None else None) for k in SEQ}
        xp, bp = prev if prev is not None else (None, None)
        ys.append(ssa.ssm_step3(state, tok["x"], tok["delta"], tok["lam"], t["Are"], t["theta"], tok["Bm"],
                                tok["Cm"], D=t.get("D"), z=tok["z"], x_prev=xp, B_prev=bp))
        prev = (tok["x"], tok["Bm"])
    torch.cuda.synchronize()
    return torch.stack(ys, dim=1)


def _start(w):
    st = torch.from_numpy(np.ascontiguousarray(w["h0"])).to(DEV) if w.get("h0") is not None else \
        torch.zeros((w["x"].shape[0], w["x"].shape[2], w["Are"].shape[1], 2), dtype=torch.float32, device=DEV)
    prev = None
    if w.get("x_prev") is not None:
        prev = (si.to_torch(w["x_prev"], DEV), si.to_torch(w["B_prev"], DEV))
    return st, prev


SMALL = [
    # B, D, N, dtype, with_D, with_z, with_h0, with_prev
    (1, 64, 16, si.F32, True, True, True, True),
    (2, 70, 4, si.BF16, True, False, True, False),
    (3, 130, 8, si.F32, False, True, False, True),
    (1, 1, 32, si.BF16, True, True, True, True),
    (2, 96, 64, si.BF16, True, True, True, True),
    (1, 33, 128, si.F32, False, False, True, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_D{}_N{}_{}_D{}z{}h{}p{}".format(*c))
def test_step3_one_token(case):
    B, D, N, dt, wd, wz, wh, wp = case
    print(f"[step3] {case}", flush=True)
    w = si.scan3_inputs(B, 1, D, N, dtype=dt, seed=61, with_D=wd, with_z=wz, with_h0=wh, with_prev=wp)
    st, prev = _start(w)
    y = gpu_steps(w, 0, 1, st, prev)
    yr, hr = oracle_scan3(w)
    compare(out_f64(y), yr, storage(w), what=f"{case} y")
    compare(out_f64(st), hr, "f32", what=f"{case} state")


@pytest.mark.parametrize("case", [(3, 50, 200, 16, si.BF16), (2, 20, 64, 64, si.F32), (1, 40, 70, 4, si.BF16)],
                         ids=lambda c: "B{}_T{}_D{}_N{}_{}".format(*c))
def test_step3_chain_equals_scan(case):
    """T steps, each given the token before it, equal the oracle's scan over the T
    tokens from the same state and previous token: y at every step, the final state."""
    B, T, D, N, dt = case
    print(f"[step3 chain] {case}", flush=True)
    w = si.scan3_inputs(B, T, D, N, dtype=dt, seed=62, with_h0=True, with_prev=True)
    st, prev = _start(w)
    y = gpu_steps(w, 0, T, st, prev)
    yr, hr = oracle_scan3(w)
    compare(out_f64(y), yr, storage(w), what=f"{case} y")
    compare(out_f64(st), hr, "f32", what=f"{case} state")


def test_step3_prefill_then_steps():
    """ssm_scan3_fwd over L tokens, then S steps handing over the last token, equals the
    oracle's scan over L + S tokens."""
    B, L, S, D, N = 2, 300, 6, 128, 16
    w = si.scan3_inputs(B, L + S, D, N, dtype=si.BF16, seed=63, with_h0=True, with_prev=True)
    pre = {k: (np.ascontiguousarray(v[:, :L]) if k in SEQ and v is not None else v) for k, v in w.items()}
    y0, hf = gpu_scan3(pre)
    tl = _dev(w)
    prev = (tl["x"][:, L - 1].clone(), tl["Bm"][:, L - 1].clone())
    st = hf.clone()
    y1 = gpu_steps(w, L, L + S, st, prev)
    yr, hr = oracle_scan3(w)
    compare(out_f64(torch.cat([y0, y1], dim=1)), yr, "bf16", what="prefill + steps y")
    compare(out_f64(st), hr, "f32", what="prefill + steps state")


def test_step3_decode_layer_100_steps():
    """A Mamba-790m-sized decode layer (B=64, D=3072, N=16, bf16) chained over 100 steps
    in place: y at every step and the final state against the oracle's scan."""
    B, T, D, N = 64, 100, 3072, 16
    print(f"[step3] B{B} D{D} N{N} x{T}", flush=True)
    w = si.scan3_inputs(B, T, D, N, dtype=si.BF16, seed=64, with_h0=True, with_prev=True)
    st, prev = _start(w)
    y = gpu_steps(w, 0, T, st, prev)
    yr, hr = oracle_scan3(w)
    compare(out_f64(y), yr, "bf16", what="decode layer y")
    compare(out_f64(st), hr, "f32", what="decode layer state")


def test_step3_hip_graph_replay_matches_eager():
    """Four steps captured in a HIP graph and replayed (eager work and synchronisations
    between replays) equal the same steps run eagerly, bit for bit, every replay."""
    B, T, D, N = 4, 4, 256, 16
    w = si.scan3_inputs(B, T, D, N, dtype=si.BF16, seed=65, with_h0=True, with_prev=True)
    t = _dev(w)
    toks = [{k: t[k][:, s].clone() for k in SEQ} for s in range(T)]
    xp0, bp0 = t["x_prev"], t["B_prev"]
    st0 = t["h0"].clone()

    def run(state, ys):
        prev = (xp0, bp0)
        for s in range(T):
            ssa.ssm_step3(state, toks[s]["x"], toks[s]["delta"], toks[s]["lam"], t["Are"], t["theta"],
                          toks[s]["Bm"], toks[s]["Cm"], D=t["D"], z=toks[s]["z"], x_prev=prev[0], B_prev=prev[1],
                          y=ys[s])
            prev = (toks[s]["x"], toks[s]["Bm"])

    ref_state = st0.clone()
    ref_y = [torch.empty((B, D), dtype=torch.bfloat16, device=DEV) for _ in range(T)]
    run(ref_state, ref_y)
    torch.cuda.synchronize()
    g_state = st0.clone()
    g_y = [torch.empty((B, D), dtype=torch.bfloat16, device=DEV) for _ in range(T)]
    graph = torch.cuda.CUDAGraph()
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        with torch.cuda.graph(graph, stream=s_):
            run(g_state, g_y)
    torch.cuda.current_stream().wait_stream(s_)
    torch.cuda.synchronize()
    for rep in range(3):
        g_state.copy_(st0)
        for s in range(T):
            g_y[s].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_state, ref_state), rep
        for s in range(T):
            assert torch.equal(g_y[s], ref_y[s]), (rep, s)
        _ = (torch.randn(1024, device=DEV) * 2).sum().item()  # eager work between replays
