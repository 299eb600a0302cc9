"""GPU parity of ssm_ssd_fwd (Mamba-2 SSD chunked scan) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import selective_scan_amd as ssa
import ssm_inputs as si
from gpu_util import DEV, out_f64
from parity import compare

pytestmark = pytest.mark.gpu


def gpu_ssd(w, chunk, **kw):
    t = {k: (si.to_torch(w[k], DEV) if w.get(k) is not None else None)
         for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    y, hf = ssa.ssm_ssd_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"],
                            h0=t["h0"], chunk=chunk, **kw)
    torch.cuda.synchronize()
    return y, hf


def oracle_ssd(w, hsel=None):
    f = {k: si.to_f64(w[k]) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    if hsel is not None:
        f["x"] = np.ascontiguousarray(f["x"][:, :, hsel])
        f["delta"] = np.ascontiguousarray(f["delta"][:, :, hsel])
        f["A"] = np.ascontiguousarray(f["A"][hsel])
        if f["z"] is not None:
            f["z"] = np.ascontiguousarray(f["z"][:, :, hsel])
        if f["D"] is not None:
            f["D"] = np.ascontiguousarray(f["D"][hsel])
        if f["h0"] is not None:
            f["h0"] = np.ascontiguousarray(f["h0"][:, hsel])
    return oracle.ssd_seq(f["x"], f["delta"], f["A"], f["Bm"], f["Cm"], D=f["D"], z=f["z"], h0=f["h0"])


def _check(w, chunk, hsel=None, what=""):
    y, hf = gpu_ssd(w, chunk)
    yr, hr = oracle_ssd(w, hsel)
    yg, hg = out_f64(y), out_f64(hf)
    if hsel is not None:
        yg, hg = yg[:, :, hsel], hg[:, hsel]
    compare(yg, yr, "bf16", what=f"{what} y")
    compare(hg, hr, "f32", what=f"{what} h_final")


SMALL = [
    # B, L, H, N, chunk, D, z, h0
    (1, 32, 1, 64, 32, False, False, False),
    (2, 100, 3, 64, 32, True, True, True),
    (1, 300, 2, 128, 64, True, False, True),
    (2, 257, 2, 128, 256, False, True, False),
    (1, 1000, 3, 128, 128, True, True, True),
    (3, 96, 2, 64, 64, True, True, True),
    (1, 1, 2, 128, 256, True, True, True),
    (1, 2100, 2, 64, 96, True, True, True),
    (1, 800, 2, 128, 192, True, True, True),
    (2, 700, 1, 64, 224, False, True, True),
    (1, 650, 2, 128, 160, True, False, True),
    # chunks that are not a multiple of 32: tiled as the next multiple, the rows
    # past a chunk's end (the next chunk's) masked
    (1, 300, 2, 128, 1, True, True, True),
    (2, 257, 2, 64, 7, True, False, True),
    (1, 90, 1, 64, 33, False, True, False),
    (1, 500, 3, 128, 50, True, True, True),
    (1, 1000, 2, 64, 100, True, True, False),
    (2, 700, 2, 128, 200, False, True, True),
    (1, 513, 2, 128, 255, True, True, True),
    # chunks above 256 steps run as 256-step chunks (the same recurrence)
    (1, 700, 2, 128, 300, True, True, True),
    (2, 1100, 1, 64, 512, False, True, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_L{}_H{}_N{}_Q{}_D{}z{}h{}".format(*c))
def test_ssd_small_shapes(case):
    B, L, H, N, Q, wd, wz, wh = case
    print(f"[ssd small] {case}", flush=True)
    w = si.ssd_inputs(B, L, H, 64, N, seed=21, with_D=wd, with_z=wz, with_h0=wh)
    _check(w, Q, what=str(case))


def test_ssd_empty_sequence():
    w = si.ssd_inputs(2, 0, 3, 64, 128, seed=1, with_h0=True)
    y, hf = gpu_ssd(w, 256)
    assert y.shape == (2, 0, 3, 64)
    np.testing.assert_array_equal(out_f64(hf), w["h0"].astype(np.float64))


@pytest.mark.parametrize("L,Q", [(8192, 256), (8192, 64), (8000, 256), (8000, 64)])
def test_ssd_config_bf16_B4_H24_P64_N128(L, Q):
    """The SSD workload at every (L, chunk) pair, every head and element against
    the sequential oracle."""
    print(f"[ssd] bf16 B4 L{L} H24 P64 N128 Q{Q} (every head)", flush=True)
    w = si.ssd_inputs(4, L, 24, 64, 128, seed=0)
    _check(w, Q, what=f"c3 L{L} Q{Q}")


def test_ssd_matches_mamba1_scan_mapping_on_gpu():
    """SSD == Mamba-1 scan with D = H*P channels (A and Delta repeated per head)."""
    B, L, H, P, N = 2, 700, 2, 64, 64
    w = si.ssd_inputs(B, L, H, P, N, seed=4, with_D=True, with_z=True, with_h0=True)
    ys, hs = gpu_ssd(w, 64)
    x = w["x"].reshape(B, L, H * P)
    m = dict(x=x, delta=np.ascontiguousarray(np.repeat(w["delta"], P, axis=2)), z=w["z"].reshape(B, L, H * P),
             Bm=w["Bm"], Cm=w["Cm"],
             A=np.ascontiguousarray(np.repeat(w["A"], P)[:, None] * np.ones((1, N), np.float32)),
             D=np.ascontiguousarray(np.repeat(w["D"], P)),
             h0=np.ascontiguousarray(w["h0"].transpose(0, 1, 3, 2).reshape(B, H * P, N)), dtype=si.BF16)
    from gpu_util import gpu_scan
    ym, hm = gpu_scan(m)
    hs_t = out_f64(hs).transpose(0, 1, 3, 2).reshape(B, H * P, N)
    compare(hs_t, out_f64(hm), "f32", tol=1e-4, what="ssd vs scan h_final")
    yr, _ = oracle_ssd(w)
    compare(out_f64(ys), yr, "bf16", what="ssd y")
    compare(out_f64(ym).reshape(B, L, H, P), yr, "bf16", what="scan-as-ssd y")


def test_ssd_deterministic():
    w = si.ssd_inputs(2, 2000, 4, 64, 128, seed=5, with_D=True, with_z=True, with_h0=True)
    y1, h1 = gpu_ssd(w, 256)
    y2, h2 = gpu_ssd(w, 256)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_ssd_tensors_beyond_2GiB():
    """Maximum-size edge: B=16, L=2^16 + 100 (ragged last chunk), H=24, P=64, N=128,
    chunk 256, bf16, so x and y hold 3.2 GB each and the later batch rows start past
    2 GiB. The inputs repeat a seeded block of 1024 steps along L; the oracle runs on
    the first and last batch rows and two heads over the whole sequence."""
    B, Lb, L, H, P, N = 16, 1024, (1 << 16) + 100, 24, 64, 128
    print(f"[ssd] bf16 B{B} L{L} H{H} N{N} (> 2 GiB per tensor)", flush=True)
    w = si.ssd_inputs(B, Lb, H, P, N, seed=24, with_D=True, with_z=True, with_h0=True)
    reps = -(-L // Lb)
    t = {k: si.to_torch(w[k], DEV) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    big = {}
    for k in ("x", "delta", "z", "Bm", "Cm"):
        v = t[k]
        big[k] = v.repeat(1, reps, *([1] * (v.dim() - 2)))[:, :L].contiguous()
    assert big["x"].numel() * 2 > (1 << 31)
    y, hf = ssa.ssm_ssd_fwd(big["x"], big["delta"], t["A"], big["Bm"], big["Cm"], D=t["D"], z=big["z"], h0=t["h0"],
                            chunk=256)
    torch.cuda.synchronize()
    bsel, hsel = np.array([0, B - 1]), np.array([0, H - 1])
    yg = out_f64(y[torch.from_numpy(bsel).to(DEV)][:, :, torch.from_numpy(hsel).to(DEV)].contiguous())
    hg = out_f64(hf)[bsel][:, hsel]
    del big, y
    torch.cuda.empty_cache()
    f = {k: si.to_f64(w[k]) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}

    def tile(a):
        a = a[bsel]
        return np.ascontiguousarray(np.tile(a, (1, reps) + (1,) * (a.ndim - 2))[:, :L])
    yr, hr = oracle.ssd_seq(tile(f["x"][:, :, hsel]), tile(f["delta"][:, :, hsel]), np.ascontiguousarray(f["A"][hsel]),
                            tile(f["Bm"]), tile(f["Cm"]), D=np.ascontiguousarray(f["D"][hsel]),
                            z=tile(f["z"][:, :, hsel]), h0=np.ascontiguousarray(f["h0"][bsel][:, hsel]))
    compare(yg, yr, "bf16", what="beyond 2 GiB y")
    compare(hg, hr, "f32", what="beyond 2 GiB h_final")
