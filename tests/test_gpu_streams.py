"""Calls launched on a side stream while the default stream allocates and
overwrites memory: the binding's outputs and workspace must belong to the launch
stream, so the caching allocator cannot hand their blocks to the default stream
while the kernels still use them. Results must equal a plain default-stream call."""
import pytest
import torch

import selective_scan_amd as ssa
import ssm_inputs as si
from gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu


def _churn(nbytes, rounds=6):
    """Default-stream allocations of the given size, filled with NaN bit patterns."""
    keep = []
    for _ in range(rounds):
        t = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=DEV)
        t.fill_(float("nan"))
        keep.append(t)
        del t
    return keep


def test_scan_ssd_bwd_on_side_stream():
    side = torch.cuda.Stream()
    # Mamba-1 scan (several segment groups, so the workspace is used)
    w = si.scan_inputs(2, 4096, 256, 16, dtype=si.BF16, seed=31, with_h0=True)
    t = to_dev(w, ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0"))
    y_ref, h_ref = ssa.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"], h0=t["h0"])
    # SSD
    s = si.ssd_inputs(2, 1500, 3, 64, 128, seed=32, with_D=True, with_z=True, with_h0=True)
    u = to_dev(s, ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0"))
    ys_ref, hs_ref = ssa.ssm_ssd_fwd(u["x"], u["delta"], u["A"], u["Bm"], u["Cm"], D=u["D"], z=u["z"],
                                     h0=u["h0"], chunk=64)
    # backward
    gw = si.scan_grad_inputs(2, 4096, 256, 16, dtype=si.BF16, seed=33)
    g = to_dev(gw, ("dy", "dh_final"))
    gb_ref = ssa.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], g["dy"], D=t["D"], z=t["z"],
                              h0=t["h0"], dh_final=g["dh_final"])
    torch.cuda.synchronize()

    side.wait_stream(torch.cuda.current_stream())
    y, h = ssa.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"], h0=t["h0"],
                            stream=side)
    junk = _churn(ssa.ssm_scan_workspace_size(2, 4096, 256, 16))
    ys, hs = ssa.ssm_ssd_fwd(u["x"], u["delta"], u["A"], u["Bm"], u["Cm"], D=u["D"], z=u["z"], h0=u["h0"],
                             chunk=64, stream=side)
    junk += _churn(ssa.ssm_ssd_workspace_size(2, 1500, 3, 64, 128, 64))
    gb = ssa.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], g["dy"], D=t["D"], z=t["z"],
                          h0=t["h0"], dh_final=g["dh_final"], stream=side)
    junk += _churn(ssa.ssm_scan_bwd_workspace_size(2, 4096, 256, 16))
    torch.cuda.synchronize()
    del junk
    assert torch.equal(y, y_ref) and torch.equal(h, h_ref)
    assert torch.equal(ys, ys_ref) and torch.equal(hs, hs_ref)
    for k, v in gb_ref.items():
        if v is not None:
            assert torch.equal(gb[k], v), k
