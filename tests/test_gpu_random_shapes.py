"""GPU parity on shapes drawn at random (fixed seeds) beside the hand-picked ones:
the scan, the SSD forward (chunk lengths, head counts, ragged tails, super-chunk
splits), the scan's backward pass, the scan with its discretisation options, the
Mamba-3 scan, and chains of the three decode steps, each against the fp64 oracle
on the same stored inputs."""
import numpy as np
import pytest

import ssm_inputs as si
from gpu_util import gpu_scan_bwd, oracle_scan_bwd, out_f64, storage
from parity import compare

pytestmark = pytest.mark.gpu


def _draw(n, seed, make):
    rng = np.random.default_rng(seed)
    return [make(rng) for _ in range(n)]


def _flags(rng, k):
    return tuple(bool(rng.integers(0, 2)) for _ in range(k))


SSD_CASES = _draw(30, 2024, lambda r: (int(r.integers(1, 4)), int(r.integers(1, 2500)), int(r.integers(1, 5)),
                                       int(r.choice([64, 128])), int(r.choice([32, 64, 96, 128, 160, 192, 224, 256])))
                  + _flags(r, 3))
# chunk lengths anywhere in [1, 256], mostly not multiples of 32
SSD_ANY_CHUNK = _draw(24, 2027, lambda r: (int(r.integers(1, 3)), int(r.integers(1, 1500)), int(r.integers(1, 4)),
                                          int(r.choice([64, 128])), int(r.integers(1, 257))) + _flags(r, 3))
BWD_CASES = _draw(30, 2025, lambda r: (int(r.integers(1, 4)), int(r.integers(1, 3000)), int(r.integers(1, 300)),
                                       int(r.choice([4, 8, 16, 32, 64, 128, 256])), bool(r.integers(0, 2)))
                  + _flags(r, 4))
VAR_CASES = _draw(24, 2026, lambda r: (int(r.integers(1, 3)), int(r.integers(1, 2000)), int(r.integers(1, 200)),
                                      int(r.choice([4, 8, 16, 32, 64, 128, 256])), bool(r.integers(0, 2)),
                                      str(r.choice(["euler", "zoh"])), bool(r.integers(0, 2))))


@pytest.mark.parametrize("case", SSD_CASES, ids=lambda c: "B{}_L{}_H{}_N{}_Q{}_D{}z{}h{}".format(*c))
def test_ssd_random_shapes(case):
    import test_gpu_ssd as T
    B, L, H, N, Q, wd, wz, wh = case
    print(f"[ssd random] {case}", flush=True)
    w = si.ssd_inputs(B, L, H, 64, N, dtype=si.BF16, seed=L, with_D=wd, with_z=wz, with_h0=wh)
    T._check(w, Q, what=str(case))


@pytest.mark.parametrize("case", SSD_ANY_CHUNK, ids=lambda c: "B{}_L{}_H{}_N{}_Q{}_D{}z{}h{}".format(*c))
def test_ssd_random_chunk_lengths(case):
    import test_gpu_ssd as T
    B, L, H, N, Q, wd, wz, wh = case
    print(f"[ssd random chunk] {case}", flush=True)
    w = si.ssd_inputs(B, L, H, 64, N, dtype=si.BF16, seed=L + 7, with_D=wd, with_z=wz, with_h0=wh)
    T._check(w, Q, what=str(case))


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}_L{}_D{}_N{}_bf{}_D{}z{}h{}g{}".format(*c))
def test_scan_bwd_random_shapes(case):
    B, L, D, N, bf, wd, wz, wh, wg = case
    print(f"[scan_bwd random] {case}", flush=True)
    dt = si.BF16 if bf else si.F32
    w = si.scan_inputs(B, L, D, N, dtype=dt, seed=L, with_D=wd, with_z=wz, with_h0=wh)
    gw = si.scan_grad_inputs(B, L, D, N, dtype=dt, seed=L + 1, with_dh_final=wg)
    g, r, st = gpu_scan_bwd(w, gw), oracle_scan_bwd(w, gw), storage(w)
    for k in ("dx", "ddelta", "dz", "dBm", "dCm", "dA", "dD", "dh0"):
        if r.get(k) is None:
            assert g.get(k) is None
            continue
        compare(out_f64(g[k]), r[k], st if k in ("dx", "ddelta", "dz", "dBm", "dCm") else "f32",
                what=f"{case} {k}")


@pytest.mark.parametrize("case", VAR_CASES, ids=lambda c: "B{}_L{}_D{}_N{}_bf{}_{}_sp{}".format(*c))
def test_scan_variant_random_shapes(case):
    import test_gpu_scan_var as V
    B, L, D, N, bf, disc, sp = case
    print(f"[scan variant random] {case}", flush=True)
    dt = si.BF16 if bf else si.F32
    w, bias = V._inputs(B, L, D, N, dt, L, True, True, True, True, softplus=sp)
    (y, hf), (yr, hr) = V._run(w, bias, disc, sp)
    compare(out_f64(y), yr, storage(w), what=f"{case} y")
    compare(out_f64(hf), hr, "f32", what=f"{case} h_final")


SCAN_CASES = _draw(40, 2027, lambda r: (int(r.integers(1, 4)), int(r.integers(1, 5000)), int(r.integers(1, 400)),
                                        int(r.choice([4, 8, 16, 32, 64, 128, 256])), bool(r.integers(0, 2)))
                   + _flags(r, 3))
SCAN3_CASES = _draw(20, 2028, lambda r: (int(r.integers(1, 4)), int(r.integers(1, 3000)), int(r.integers(1, 300)),
                                        int(r.choice([4, 8, 16])), bool(r.integers(0, 2))) + _flags(r, 4))
STEP3_CASES = _draw(12, 2029, lambda r: (int(r.integers(1, 5)), int(r.integers(1, 40)), int(r.integers(1, 300)),
                                        int(r.choice([4, 8, 16, 32, 64, 128])), bool(r.integers(0, 2))))


@pytest.mark.parametrize("case", SCAN_CASES, ids=lambda c: "B{}_L{}_D{}_N{}_bf{}_D{}z{}h{}".format(*c))
def test_scan_random_shapes(case):
    import test_gpu_scan as S
    B, L, D, N, bf, wd, wz, wh = case
    print(f"[scan random] {case}", flush=True)
    w = si.scan_inputs(B, L, D, N, dtype=si.BF16 if bf else si.F32, seed=L, with_D=wd, with_z=wz, with_h0=wh)
    S._check(w, what=str(case))


@pytest.mark.parametrize("case", SCAN3_CASES, ids=lambda c: "B{}_L{}_D{}_N{}_bf{}_D{}z{}h{}p{}".format(*c))
def test_scan3_random_shapes(case):
    import test_gpu_scan3 as S3
    B, L, D, N, bf, wd, wz, wh, wp = case
    print(f"[scan3 random] {case}", flush=True)
    w = si.scan3_inputs(B, L, D, N, dtype=si.BF16 if bf else si.F32, seed=L, with_D=wd, with_z=wz, with_h0=wh,
                        with_prev=wp)
    S3._check(w, str(case))


@pytest.mark.parametrize("case", STEP3_CASES, ids=lambda c: "B{}_T{}_D{}_N{}_bf{}".format(*c))
def test_step3_random_chains(case):
    import test_gpu_step3 as T3
    B, T, D, N, bf = case
    print(f"[step3 random] {case}", flush=True)
    w = si.scan3_inputs(B, T, D, N, dtype=si.BF16 if bf else si.F32, seed=T, with_h0=True, with_prev=True)
    st, prev = T3._start(w)
    y = T3.gpu_steps(w, 0, T, st, prev)
    yr, hr = T3.oracle_scan3(w)
    compare(out_f64(y), yr, storage(w), what=f"{case} y")
    compare(out_f64(st), hr, "f32", what=f"{case} state")


STEP_CASES = _draw(12, 2030, lambda r: (int(r.integers(1, 5)), int(r.integers(1, 400)),
                                        int(r.choice([4, 8, 16, 32, 64, 128, 256])), bool(r.integers(0, 2)))
                   + _flags(r, 2))
SSD_STEP_CASES = _draw(10, 2031, lambda r: (int(r.integers(1, 4)), int(r.integers(1, 6)),
                                            int(r.choice([16, 32, 64, 128, 256])), bool(r.integers(0, 2)))
                       + _flags(r, 2))


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "B{}_D{}_N{}_bf{}_D{}z{}".format(*c))
def test_step_random_chains(case):
    """Eight chained Mamba-1 decode steps in place against the oracle's steps."""
    import test_gpu_step as ST
    B, D, N, bf, wd, wz = case
    print(f"[step random] {case}", flush=True)
    ST._run_steps(si.step_inputs(B, D, N, 8, dtype=si.BF16 if bf else si.F32, seed=D, with_D=wd, with_z=wz), 8)


@pytest.mark.parametrize("case", SSD_STEP_CASES, ids=lambda c: "B{}_H{}_N{}_bf{}_D{}z{}".format(*c))
def test_ssd_step_random_chains(case):
    """Six chained Mamba-2 decode steps in place against the oracle's steps."""
    import test_gpu_ssd_step as SST
    B, H, N, bf, wd, wz = case
    print(f"[ssd step random] {case}", flush=True)
    SST._run_steps(si.ssd_step_inputs(B, H, 64, N, 6, dtype=si.BF16 if bf else si.F32, seed=H + 3, with_D=wd,
                                      with_z=wz), 6)
