"""The measurement kernels of the library (not the scan itself): the copy the HBM
byte counters are calibrated with, the in-place streaming kernel the decode steps
are compared with, and the VALU issue-rate probes, checked for what they compute."""
import pytest
import torch

import selective_scan_amd as ssa
from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [4, 4 * 1000 + 4, (1 << 22) + 12])
def test_diag_copy_and_scale(n):
    g = torch.Generator(device="cpu").manual_seed(n)
    src = torch.randn(n, generator=g).to(DEV)
    dst = torch.full_like(src, float("nan"))
    ssa.ssm_diag_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    ssa.ssm_diag_stream_scale(dst, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(dst, src * 0.5)  # a power-of-two scale is exact


def test_diag_valu_rate_probe_values():
    """The probes' chains stay in range ([0.5, 1], the sin and cos chains in [-1, 1]) and
    the modes compute what they say:
    the fma chain's fixed point is 0.75; the outputs are finite."""
    out = torch.empty(2 * 256, dtype=torch.float32, device=DEV)
    for mode in (0, 1, 2, 3, 4):
        ssa.ssm_diag_valu_rate(mode, out, 64)
        torch.cuda.synchronize()
        v = out / 8.0  # each lane sums its 8 chains
        lo = -1.0 if mode >= 3 else 0.5  # the sin and cos chains live in [-1, 1]
        assert torch.isfinite(out).all() and bool((v >= lo).all()) and bool((v <= 1.0).all()), mode
        if mode == 1:
            assert torch.allclose(v, torch.full_like(v, 0.75), atol=1e-6)
