"""GPU parity of ssm_scan_bwd (gradient of the Mamba-1 scan) against the fp64
oracle's reverse-mode gradient, on the same stored inputs and cotangents."""
import numpy as np
import pytest
import torch

import ssm_inputs as si
from gpu_util import gpu_scan_bwd, oracle_scan_bwd, out_f64, storage
from parity import compare

pytestmark = pytest.mark.gpu

PER_CHANNEL = ("dx", "ddelta", "dz")   # [B, L, D], io dtype
SHARED = ("dBm", "dCm")                # [B, L, N], io dtype, summed over channels
PARAMS = ("dA", "dD", "dh0")           # fp32


def _check(w, gw, what="", sel=None, keys=None):
    g = gpu_scan_bwd(w, gw)
    r = oracle_scan_bwd(w, gw, sel)
    st = storage(w)
    for k in keys or (PER_CHANNEL + SHARED + PARAMS):
        if r.get(k) is None:
            assert g.get(k) is None, f"{what}: {k} returned without its input"
            continue
        v = out_f64(g[k])
        if sel is not None:
            if k in PER_CHANNEL:
                v = v[:, :, sel]
            elif k in ("dA", "dD"):
                v = v[sel]
            elif k == "dh0":
                v = v[:, sel]
        compare(v, r[k], st if k in PER_CHANNEL + SHARED else "f32", what=f"{what} {k}")


SMALL = [
    # B, L, D, N, dtype, with_D, with_z, with_h0, with_dh_final
    (1, 1, 64, 16, si.F32, True, True, True, True),
    (2, 37, 70, 16, si.BF16, True, True, True, True),
    (1, 300, 64, 4, si.F32, False, False, False, False),
    (3, 1000, 130, 8, si.BF16, True, False, True, True),
    (1, 2001, 32, 16, si.F32, True, True, False, True),
    (2, 513, 200, 16, si.BF16, True, True, True, False),
    (1, 4097, 96, 16, si.BF16, False, True, False, True),
    (5, 77, 1, 16, si.F32, True, True, True, True),
    (1, 6, 64, 8, si.BF16, True, True, True, True),
    (2, 999, 64, 4, si.BF16, True, True, True, True),
    # N >= 32: chunks of 16 states, partial sums over n added across the chunks
    (2, 300, 70, 32, si.BF16, True, True, True, True),
    (1, 1000, 96, 64, si.F32, False, True, False, True),
    (3, 257, 130, 128, si.BF16, True, False, True, False),
    (1, 129, 64, 256, si.F32, True, True, True, True),
    (2, 5, 33, 64, si.BF16, False, False, False, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_L{}_D{}_N{}_{}_D{}z{}h{}g{}".format(*c))
def test_scan_bwd_small_shapes(case):
    B, L, D, N, dt, wd, wz, wh, wg = case
    print(f"[scan_bwd small] {case}", flush=True)
    w = si.scan_inputs(B, L, D, N, dtype=dt, seed=7, with_D=wd, with_z=wz, with_h0=wh)
    gw = si.scan_grad_inputs(B, L, D, N, dtype=dt, seed=8, with_dh_final=wg)
    _check(w, gw, what=str(case))


def test_scan_bwd_empty_sequence():
    w = si.scan_inputs(2, 0, 64, 16, dtype=si.BF16, seed=1, with_h0=True)
    gw = si.scan_grad_inputs(2, 0, 64, 16, dtype=si.BF16, seed=2)
    g = gpu_scan_bwd(w, gw)
    np.testing.assert_array_equal(out_f64(g["dh0"]), gw["dh_final"].astype(np.float64))
    assert not torch.any(g["dA"]) and not torch.any(g["dD"])
    assert g["dx"].shape == (2, 0, 64) and g["dBm"].shape == (2, 0, 16)


def test_scan_bwd_headline_layer_all_outputs():
    """The headline layer (B=1, L=4096, D=1536, N=16, bf16): every output in full."""
    print("[scan_bwd] bf16 B1 L4096 D1536 N16", flush=True)
    w = si.scan_inputs(1, 4096, 1536, 16, dtype=si.BF16, seed=0)
    gw = si.scan_grad_inputs(1, 4096, 1536, 16, dtype=si.BF16, seed=0)
    _check(w, gw, what="B1 L4096 D1536")


@pytest.mark.parametrize("N", [32, 64, 128, 256])
def test_scan_bwd_state_dim_sweep_all_outputs(N):
    """The state-dimension sweep shape (B=1, L=4096, D=1536, bf16) at N = 32, 64,
    128, 256: every output in full."""
    print(f"[scan_bwd] bf16 B1 L4096 D1536 N{N}", flush=True)
    w = si.scan_inputs(1, 4096, 1536, N, dtype=si.BF16, seed=0)
    gw = si.scan_grad_inputs(1, 4096, 1536, N, dtype=si.BF16, seed=0)
    _check(w, gw, what=f"B1 L4096 D1536 N{N}")


def test_scan_bwd_training_shape_all_outputs():
    """The training-step sweep's largest shape (B=8, L=32768, D=512, N=16, bf16),
    in the launch configuration the benchmark times: every output in full."""
    print("[scan_bwd] bf16 B8 L32768 D512 N16", flush=True)
    w = si.scan_inputs(8, 32768, 512, 16, dtype=si.BF16, seed=0)
    gw = si.scan_grad_inputs(8, 32768, 512, 16, dtype=si.BF16, seed=0)
    _check(w, gw, what="B8 L32768 D512")


def test_scan_bwd_deterministic():
    w = si.scan_inputs(2, 1500, 100, 16, dtype=si.BF16, seed=3, with_h0=True)
    gw = si.scan_grad_inputs(2, 1500, 100, 16, dtype=si.BF16, seed=4)
    g1 = gpu_scan_bwd(w, gw)
    g2 = gpu_scan_bwd(w, gw)
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g2[k]), k


def test_scan_bwd_long_sequence_few_channels():
    """B=1, L=20000, D=64, N=16: 1250 segments in 313 groups, so both carries walk
    quarters longer than they keep in registers (the re-read path)."""
    print("[scan_bwd] B1 L20000 D64 N16 (long group walk)", flush=True)
    w = si.scan_inputs(1, 20000, 64, 16, dtype=si.BF16, seed=10, with_h0=True)
    gw = si.scan_grad_inputs(1, 20000, 64, 16, dtype=si.BF16, seed=11)
    _check(w, gw, what="long walk")


def test_scan_bwd_without_dh0_changes_nothing_else():
    """dh0 not requested (NULL): every other gradient is bit-identical."""
    w = si.scan_inputs(2, 700, 96, 16, dtype=si.BF16, seed=12, with_h0=True)
    gw = si.scan_grad_inputs(2, 700, 96, 16, dtype=si.BF16, seed=13)
    g1 = gpu_scan_bwd(w, gw)
    g2 = gpu_scan_bwd(w, gw, want_dh0=False)
    assert g2["dh0"] is None
    for k, v in g1.items():
        if k != "dh0":
            assert torch.equal(v, g2[k]), k


def test_scan_bwd_tensors_beyond_2GiB():
    """Maximum-size edge: B=1, L=2^20 + 37 (ragged), D=2048, N=16, bf16, so x, Delta, z,
    dy and the per-channel gradients each hold 4.3 GB (the checkpoints 34 GB). The
    inputs repeat a seeded block of 4096 steps along L; the oracle runs on 16 channels
    over the whole sequence (dx, ddelta, dz, dA, dD, dh0 of those channels; dB and dC
    sum over every channel and are covered by the full-size tests above)."""
    import oracle
    import selective_scan_amd as ssa
    from gpu_util import DEV, to_dev
    B, Lb, L, D, N = 1, 4096, (1 << 20) + 37, 2048, 16
    print(f"[scan_bwd] bf16 B{B} L{L} D{D} N{N} (> 2 GiB per tensor)", flush=True)
    w = si.scan_inputs(B, Lb, D, N, dtype=si.BF16, seed=25, with_h0=True)
    gw = si.scan_grad_inputs(B, Lb, D, N, dtype=si.BF16, seed=26)
    reps = -(-L // Lb)
    t = to_dev(w, ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0"))
    g = to_dev(gw, ("dy", "dh_final"))
    big = {k: t[k].repeat(1, reps, 1)[:, :L].contiguous() for k in ("x", "delta", "z", "Bm", "Cm")}
    dy = g["dy"].repeat(1, reps, 1)[:, :L].contiguous()
    assert big["x"].numel() * 2 > (1 << 31)
    out = ssa.ssm_scan_bwd(big["x"], big["delta"], t["A"], big["Bm"], big["Cm"], dy, D=t["D"], z=big["z"],
                           h0=t["h0"], dh_final=g["dh_final"])
    torch.cuda.synchronize()
    sel = np.array([0, 1, 63, 64, 500, 1023, 1024, 1500, 1919, 1920, 2000, 2040, 2045, 2046, 2047, 777])
    sd = torch.from_numpy(sel).to(DEV)
    got = {k: out_f64(out[k][:, :, sd].contiguous()) for k in ("dx", "ddelta", "dz")}
    got["dA"], got["dD"], got["dh0"] = out_f64(out["dA"])[sel], out_f64(out["dD"])[sel], out_f64(out["dh0"])[:, sel]
    del big, dy, out
    torch.cuda.empty_cache()
    tile = lambda a: np.ascontiguousarray(np.tile(a, (1, reps, 1))[:, :L])
    f = {k: si.to_f64(w[k]) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    r = oracle.scan_bwd(tile(f["x"][:, :, sel]), tile(f["delta"][:, :, sel]), np.ascontiguousarray(f["A"][sel]),
                        tile(f["Bm"]), tile(f["Cm"]), tile(si.to_f64(gw["dy"])[:, :, sel]),
                        D=np.ascontiguousarray(f["D"][sel]), z=tile(f["z"][:, :, sel]),
                        h0=np.ascontiguousarray(f["h0"][:, sel]),
                        dh_final=np.ascontiguousarray(si.to_f64(gw["dh_final"])[:, sel]))
    for k in ("dx", "ddelta", "dz"):
        compare(got[k], r[k], "bf16", what=f"beyond 2 GiB {k}")
    for k in ("dA", "dD", "dh0"):
        compare(got[k], r[k], "f32", what=f"beyond 2 GiB {k}")
