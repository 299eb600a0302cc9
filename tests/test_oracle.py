"""CPU tests of the fp64 oracle against what the mathematics fixes (no GPU).

Pins are in ``pins.py``; the hand-derived worked examples in ``golden/``.
"""
import json
import os

import numpy as np
import pytest

import pins

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def _arr(v):
    return None if v is None else np.array(v, dtype=np.float64)


def _golden(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        return json.load(f)


def test_golden_mamba1_impulse(orc):
    g = _golden("mamba1_impulse")
    i = {k: _arr(v) for k, v in g["inputs"].items()}
    y, hf = orc.scan(**i)
    np.testing.assert_allclose(y, _arr(g["expected"]["y"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(hf, _arr(g["expected"]["h_final"]), rtol=1e-13, atol=1e-15)
    yu, hu = orc.scan_unroll(**i)
    np.testing.assert_allclose(yu, _arr(g["expected"]["y"]), rtol=1e-13, atol=1e-15)


def test_golden_gated_step(orc):
    g = _golden("gated_step")
    i = {k: _arr(v) for k, v in g["inputs"].items()}
    st = i.pop("state")
    y, st2 = orc.step(st, **i)
    np.testing.assert_allclose(y, _arr(g["expected"]["y"]), rtol=1e-14)
    np.testing.assert_allclose(st2, _arr(g["expected"]["state"]), rtol=1e-14)


def test_golden_ssd_carry(orc):
    g = _golden("ssd_carry")
    i = {k: _arr(v) for k, v in g["inputs"].items()}
    ey, eh = _arr(g["expected"]["y"]), _arr(g["expected"]["h_final"])
    y, hf = orc.ssd_seq(**i)
    np.testing.assert_allclose(y, ey, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(hf, eh, rtol=1e-13, atol=1e-15)
    for q in g["chunks"]:
        y, hf = orc.ssd_chunked(**i, chunk=q)
        np.testing.assert_allclose(y, ey, rtol=1e-13, atol=1e-15, err_msg=f"chunk {q}")
        np.testing.assert_allclose(hf, eh, rtol=1e-13, atol=1e-15, err_msg=f"chunk {q}")


def test_empty_sequence(orc):
    """L = 0: no output, and the final state is the initial state."""
    p = pins.mamba1_problem(2, 0, 3, 4, seed=1)
    y, hf = orc.scan(**p)
    assert y.shape == (2, 0, 3)
    np.testing.assert_array_equal(hf, p["h0"])
    q = pins.ssd_problem(1, 0, 2, 3, 4, seed=2)
    for fn in (orc.ssd_seq, lambda **k: orc.ssd_chunked(**k, chunk=4)):
        y, hf = fn(**q)
        assert y.shape == (1, 0, 2, 3)
        np.testing.assert_array_equal(hf, q["h0"])


def test_bad_arguments_rejected(orc):
    q = pins.ssd_problem(1, 8, 1, 2, 3, seed=3)
    with pytest.raises(ValueError):
        orc.ssd_chunked(**q, chunk=0)


def test_threads_setting(orc):
    n0 = orc.get_threads()
    orc.set_threads(1)
    assert orc.get_threads() == 1
    p = pins.mamba1_problem(1, 30, 8, 4, seed=9)
    y1, _ = orc.scan(**p)
    orc.set_threads(4)
    y4, _ = orc.scan(**p)
    orc.set_threads(n0)
    np.testing.assert_array_equal(y1, y4)  # parallel only over independent channels
