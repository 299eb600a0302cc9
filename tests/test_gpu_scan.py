"""GPU parity of ssm_scan_fwd (Mamba-1 selective scan) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ssa
import ssm_inputs as si
from gpu_util import DEV, gpu_scan, oracle_scan, out_f64, storage, to_dev
from parity import compare

pytestmark = pytest.mark.gpu


def _check(w, sel=None, what=""):
    y, hf = gpu_scan(w)
    yr, hr = oracle_scan(w, sel)
    yg = out_f64(y)
    hg = out_f64(hf)
    if sel is not None:
        yg, hg = yg[:, :, sel], hg[:, sel]
    compare(yg, yr, storage(w), what=f"{what} y")
    compare(hg, hr, "f32", what=f"{what} h_final")


SMALL = [
    # B, L, D, N, dtype, with_D, with_z, with_h0
    (1, 1, 64, 16, si.F32, True, True, True),
    (2, 37, 70, 16, si.BF16, True, True, True),
    (1, 300, 64, 4, si.F32, False, False, False),
    (3, 1000, 130, 8, si.BF16, True, False, True),
    (1, 2000, 32, 32, si.F32, True, True, False),
    (2, 513, 200, 64, si.BF16, True, True, True),
    (1, 4097, 96, 16, si.BF16, False, True, False),
    (5, 77, 1, 16, si.F32, True, True, True),
    # N >= 64: the state index runs in chunks of 16 states whose C . h sums a workgroup
    # adds in LDS (two groups of eight chunks at N = 256), then a combine
    (2, 700, 90, 128, si.BF16, True, True, True),
    (1, 1500, 64, 256, si.F32, True, False, True),
    (1, 40, 33, 128, si.F32, False, True, False),
    (3, 257, 128, 256, si.BF16, True, True, False),
    # short chains run as one launch (every segment of a chain in one workgroup, the
    # carries in LDS): two to four segments, and a batch of short sequences at eight
    (3, 120, 200, 8, si.F32, True, False, True),
    (1, 100, 64, 32, si.BF16, True, True, True),
    (2, 65, 130, 4, si.BF16, False, True, True),
    (64, 256, 1536, 16, si.BF16, True, True, True),
    (16, 250, 1024, 32, si.F32, True, True, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_L{}_D{}_N{}_{}_D{}z{}h{}".format(*c))
def test_scan_small_shapes(case):
    B, L, D, N, dt, wd, wz, wh = case
    print(f"[scan small] {case}", flush=True)
    w = si.scan_inputs(B, L, D, N, dtype=dt, seed=11, with_D=wd, with_z=wz, with_h0=wh)
    _check(w, what=str(case))


def test_scan_empty_sequence_returns_initial_state():
    w = si.scan_inputs(2, 0, 64, 16, dtype=si.BF16, seed=1, with_h0=True)
    y, hf = gpu_scan(w)
    assert y.shape == (2, 0, 64)
    np.testing.assert_array_equal(out_f64(hf), w["h0"].astype(np.float64))


def test_scan_config_f32_B1_L256_D64_N16():
    print("[scan] f32 B1 L256 D64 N16", flush=True)
    w = si.scan_inputs(1, 256, 64, 16, dtype=si.F32, seed=0)
    _check(w, what="c0")


def test_scan_config_bf16_B1_L4096_D1536_N16():
    print("[scan] bf16 B1 L4096 D1536 N16 (all channels)", flush=True)
    w = si.scan_inputs(1, 4096, 1536, 16, dtype=si.BF16, seed=0)
    _check(w, what="c1")


def test_scan_config_bf16_B8_L32768_D512_N16():
    """The long-sequence workload in full: every y element (134 M) and the final state."""
    print("[scan] bf16 B8 L32768 D512 N16 (every element)", flush=True)
    w = si.scan_inputs(8, 32768, 512, 16, dtype=si.BF16, seed=0)
    _check(w, what="c2")


@pytest.mark.parametrize("N", [64, 128, 256])
def test_scan_state_dim_sweep_bf16_B1_L4096_D1536(N):
    """The state-dimension sweep (N = 64, 128, 256) at the headline layer's size,
    every channel against the oracle."""
    print(f"[scan] bf16 B1 L4096 D1536 N{N} (every channel)", flush=True)
    w = si.scan_inputs(1, 4096, 1536, N, dtype=si.BF16, seed=0)
    _check(w, what=f"N{N} sweep")


def test_scan_split_carry_on_gpu():
    """scan(x[:m]) -> h; scan(x[m:], h0=h) == scan(x)."""
    w = si.scan_inputs(2, 3000, 192, 16, dtype=si.F32, seed=5, with_h0=True)
    y, hf = gpu_scan(w)
    m = 1234
    cut = lambda a, s: None if a is None else np.ascontiguousarray(a[:, s])
    w1 = dict(w, **{k: cut(w[k], slice(0, m)) for k in ("x", "delta", "z", "Bm", "Cm")})
    y1, h1 = gpu_scan(w1)
    w2 = dict(w, **{k: cut(w[k], slice(m, None)) for k in ("x", "delta", "z", "Bm", "Cm")})
    w2["h0"] = h1.cpu().numpy()
    y2, h2 = gpu_scan(w2)
    yc = np.concatenate([out_f64(y1), out_f64(y2)], axis=1)
    compare(yc, out_f64(y), "f32", what="split y")
    compare(out_f64(h2), out_f64(hf), "f32", what="split h")


def test_scan_causality_on_gpu():
    w = si.scan_inputs(1, 2048, 128, 16, dtype=si.BF16, seed=6)
    y, _ = gpu_scan(w)
    t = 1000
    w2 = dict(w)
    for k in ("x", "delta", "z", "Bm", "Cm"):
        a = w[k].copy()
        a[:, t + 1:] = a[::-1][:, t + 1:] if a.shape[0] > 1 else np.roll(a[:, t + 1:], 1, axis=1)
        w2[k] = a
    y2, _ = gpu_scan(w2)
    a, b = out_f64(y), out_f64(y2)
    assert np.array_equal(a[:, :t + 1], b[:, :t + 1])
    assert not np.array_equal(a[:, t + 1:], b[:, t + 1:])


def test_scan_deterministic_and_ignores_workspace_contents():
    import selective_scan_amd as ssa
    w = si.scan_inputs(2, 4096, 256, 16, dtype=si.BF16, seed=7, with_h0=True)
    y1, h1 = gpu_scan(w)
    need = ssa.ssm_scan_workspace_size(2, 4096, 256, 16)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    y2, h2 = gpu_scan(w, workspace=ws)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_scan_long_sequence_few_channels():
    """B=1, L=20000, D=64: hundreds of segment groups, so the group carry walks
    quarters longer than it keeps in registers (the re-read path)."""
    print("[scan] B1 L20000 D64 N16 (long group walk)", flush=True)
    w = si.scan_inputs(1, 20000, 64, 16, dtype=si.BF16, seed=9, with_h0=True)
    _check(w, what="long walk")


def test_scan_tensors_beyond_2GiB():
    """Maximum-size edge: B=1, L=2^21 + 37 (ragged), D=1024, bf16, so x, Delta, z and y
    each hold 4.3 GB and every byte offset past 2 GiB is formed from a segment's 64-bit
    base. The inputs repeat a seeded block of 4096 steps along L (drawing 2^31 values
    per tensor would take minutes on the host); the oracle runs on 16 channels, the
    last one included, over the whole sequence."""
    B, Lb, L, D, N = 1, 4096, (1 << 21) + 37, 1024, 16
    print(f"[scan] bf16 B{B} L{L} D{D} N{N} (> 2 GiB per tensor)", flush=True)
    w = si.scan_inputs(B, Lb, D, N, dtype=si.BF16, seed=23, with_h0=True)
    reps = -(-L // Lb)
    t = to_dev(w, ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0"))
    big = {k: t[k].repeat(1, reps, 1)[:, :L].contiguous() for k in ("x", "delta", "z", "Bm", "Cm")}
    assert big["x"].numel() * 2 > (1 << 31)
    y, hf = ssa.ssm_scan_fwd(big["x"], big["delta"], t["A"], big["Bm"], big["Cm"], D=t["D"], z=big["z"],
                             h0=t["h0"])
    torch.cuda.synchronize()
    sel = np.array([0, 1, 63, 64, 127, 300, 511, 512, 640, 777, 900, 959, 960, 1000, 1022, 1023])
    yg = out_f64(y[:, :, torch.from_numpy(sel).to(DEV)].contiguous())
    hg = out_f64(hf)[:, sel]
    del big, y
    torch.cuda.empty_cache()
    tile = lambda a: np.ascontiguousarray(np.tile(a, (1, reps, 1))[:, :L])
    f = {k: si.to_f64(w[k]) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    yr, hr = oracle.scan(tile(f["x"][:, :, sel]), tile(f["delta"][:, :, sel]), np.ascontiguousarray(f["A"][sel]),
                         tile(f["Bm"]), tile(f["Cm"]), D=np.ascontiguousarray(f["D"][sel]),
                         z=tile(f["z"][:, :, sel]), h0=np.ascontiguousarray(f["h0"][:, sel]))
    compare(yg, yr, "bf16", what="beyond 2 GiB y")
    compare(hg, hr, "f32", what="beyond 2 GiB h_final")
