"""CPU tests of the seeded input generators (rounding and distributions)."""
import math

import numpy as np
import torch

import ssm_inputs as si


def test_bf16_rounding_matches_torch_rne():
    r = np.random.default_rng(0)
    v = np.concatenate([r.standard_normal(20000), r.standard_normal(2000) * 1e-20,
                        r.standard_normal(2000) * 1e20])
    v32 = v.astype(np.float32).astype(np.float64)   # fp32-representable: one rounding either way
    bits = si.round_bf16_bits(v32)
    ref = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1); 1 + 3*2^-8 -> 1 + 2^-6
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -40])
    out = si.bf16_bits_to_f64(si.round_bf16_bits(v))
    np.testing.assert_array_equal(out, [1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7])


def test_roundtrip_exact():
    r = np.random.default_rng(1)
    bits = si.round_bf16_bits(r.standard_normal(1000))
    np.testing.assert_array_equal(si.round_bf16_bits(si.bf16_bits_to_f64(bits)), bits)


def test_scan_inputs_distributions():
    w = si.scan_inputs(2, 512, 64, 16, dtype=si.BF16, seed=0)
    x = si.to_f64(w["x"])
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    d = si.to_f64(w["delta"])
    assert np.all(d > 0)
    # per-channel dt spans [1e-3, 1e-1]: the median Delta per channel follows dt
    med = np.median(d.reshape(-1, 64), axis=0)
    assert med.min() > 5e-4 and med.max() < 0.2
    b = si.to_f64(w["Bm"])
    assert abs(b.std() - 1 / math.sqrt(16)) < 0.01
    np.testing.assert_array_equal(w["A"][5], -(np.arange(16) + 1.0))
    assert w["h0"] is None and w["D"].dtype == np.float32


def test_inputs_reproducible_and_seeded():
    a = si.scan_inputs(1, 64, 8, 4, dtype=si.F32, seed=3)
    b = si.scan_inputs(1, 64, 8, 4, dtype=si.F32, seed=3)
    c = si.scan_inputs(1, 64, 8, 4, dtype=si.F32, seed=4)
    np.testing.assert_array_equal(a["x"], b["x"])
    assert not np.array_equal(a["x"], c["x"])
    assert a["x"].dtype == np.float32


def test_ssd_inputs_shapes():
    w = si.ssd_inputs(2, 100, 3, 8, 16, seed=0, with_D=True, with_z=True, with_h0=True)
    assert w["x"].shape == (2, 100, 3, 8) and w["delta"].shape == (2, 100, 3)
    assert w["Bm"].shape == (2, 100, 16) and w["h0"].shape == (2, 3, 16, 8)
    A = w["A"].astype(np.float64)
    assert np.all(A <= -1.0) and np.all(A >= -16.0)


def test_step_inputs_shapes():
    w = si.step_inputs(4, 32, 16, steps=5)
    assert w["state0"].shape == (4, 32, 16) and w["x"].shape == (5, 4, 32)
    assert abs(w["state0"].std() - 0.1) < 0.02
