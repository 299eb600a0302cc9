"""The C-ABI library: it loads, exports every declared entry point, and rejects
bad arguments before any HIP call (these run on a machine with no GPU)."""
import ctypes
import os
import re

import pytest

import selective_scan_amd as ssa
from selective_scan_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

# fake, 16-byte aligned device addresses: validation failures never dereference them
P = ctypes.c_void_p(0x10000)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ssm_scan_fwd", "ssm_scan_bwd", "ssm_ssd_fwd", "ssm_step", "ssm_ssd_step"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ops.lib()
    for name in declared_functions():
        assert hasattr(L, name), f"{name} is declared in include/ssm_scan.h but not exported"


def test_version_and_status_strings():
    L = ops.lib()
    assert L.ssm_abi_version() == 1
    assert L.ssm_status_string(0) == b"SSM_OK"
    assert L.ssm_status_string(3) == b"SSM_ERR_WORKSPACE"
    assert L.ssm_status_string(99) == b"SSM_ERR_UNKNOWN"


def _scan(B=1, L=8, D=64, N=16, io=1, x=P, delta=P, A=P, Bm=P, Cm=P, Dk=None, z=None, h0=None,
          y=P, hf=None, ws=None, wsb=0):
    return ops.lib().ssm_scan_fwd(B, L, D, N, io, x, delta, A, Bm, Cm, Dk, z, h0, y, hf, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(D=0), 1), (dict(L=-1), 1), (dict(N=0), 1), (dict(io=7), 1),
    (dict(N=12), 2), (dict(N=512), 2), (dict(B=70000), 2),
    (dict(x=None), 1), (dict(A=None), 1), (dict(y=None), 1), (dict(Cm=None), 1),
    (dict(x=ctypes.c_void_p(0x10004)), 1),
])
def test_scan_rejects_bad_arguments(kw, status):
    assert _scan(**kw) == status
    assert ops.lib().ssm_last_error().startswith(b"ssm_scan_fwd: ")


def test_scan_workspace_checks():
    need = ssa.ssm_scan_workspace_size(1, 4096, 1536, 16)
    assert need > 0
    assert _scan(L=4096, D=1536, ws=None, wsb=0) == 3
    assert _scan(L=4096, D=1536, ws=P, wsb=need - 1) == 3
    assert ssa.ssm_scan_workspace_size(1, 4096, 1536, 12) == 0
    assert ssa.ssm_scan_workspace_size(1, 32, 64, 16) == 0  # a single segment needs none
    # N = 64, 128: one workgroup holds every state chunk and finishes y itself, so a
    # single segment needs none either; N = 256 sums two chunk groups through the workspace
    assert ssa.ssm_scan_workspace_size(1, 32, 64, 64) == 0
    assert ssa.ssm_scan_workspace_size(1, 32, 64, 128) == 0
    assert ssa.ssm_scan_workspace_size(1, 32, 64, 256) > 0


def test_step_rejects_bad_arguments():
    L = ops.lib()
    ok = dict(B=2, D=64, N=16, io=1)
    def call(**kw):
        a = dict(ok, state=P, x=P, delta=P, A=P, Bm=P, Cm=P, Dk=None, z=None, y=P)
        a.update(kw)
        return L.ssm_step(a["B"], a["D"], a["N"], a["io"], a["state"], a["x"], a["delta"], a["A"],
                          a["Bm"], a["Cm"], a["Dk"], a["z"], a["y"], None)
    assert call(B=0) == 1
    assert call(N=5) == 2
    assert call(state=None) == 1
    assert call(y=ctypes.c_void_p(0x10008)) == 1
    assert call(io=3) == 1


def test_ssd_step_rejects_bad_arguments():
    L = ops.lib()
    ok = dict(B=2, H=3, Pp=64, N=128, io=1)
    def call(**kw):
        a = dict(ok, state=P, x=P, delta=P, A=P, Bm=P, Cm=P, Dk=None, z=None, y=P)
        a.update(kw)
        return L.ssm_ssd_step(a["B"], a["H"], a["Pp"], a["N"], a["io"], a["state"], a["x"], a["delta"],
                              a["A"], a["Bm"], a["Cm"], a["Dk"], a["z"], a["y"], None)
    assert call(B=0) == 1
    assert call(H=0) == 1
    assert call(io=3) == 1
    assert call(Pp=32) == 2
    assert call(N=48) == 2
    assert call(N=512) == 2
    assert call(state=None) == 1
    assert call(x=ctypes.c_void_p(0x10004)) == 1
    assert ops.lib().ssm_last_error().startswith(b"ssm_ssd_step: ")


def test_ssd_rejects_bad_arguments():
    L = ops.lib()
    def call(B=1, Lq=64, H=2, Pp=64, N=128, chunk=0, io=1, x=P):
        return L.ssm_ssd_fwd(B, Lq, H, Pp, N, chunk, io, x, P, P, P, P, None, None, None, P, None,
                             None, 0, None)
    assert call(B=0) == 1
    assert call(chunk=-1) == 1
    assert call(io=9) == 1
    assert call(io=0) == 2          # fp32 I/O not built for SSD
    assert call(Pp=32) == 2
    assert call(N=96) == 2
    assert call(B=70000) == 2


def test_python_binding_checks_tensors_before_calling():
    import torch
    x = torch.zeros(1, 4, 8)  # CPU tensors: the binding checks shapes/dtypes first
    with pytest.raises(TypeError):
        ssa.ssm_scan_fwd(x.to(torch.float64), x, torch.zeros(8, 16), torch.zeros(1, 4, 16),
                         torch.zeros(1, 4, 16))


def _bwd(B=1, L=64, D=64, N=16, io=1, Dk=None, z=None, dD=None, dz=None, ws=P, wsb=1 << 30, **kw):
    a = dict(x=P, delta=P, A=P, Bm=P, Cm=P, h0=None, dy=P, dhf=None, dx=P, ddelta=P, dA=P, dBm=P,
             dCm=P, dh0=None)
    a.update(kw)
    return ops.lib().ssm_scan_bwd(B, L, D, N, io, a["x"], a["delta"], a["A"], a["Bm"], a["Cm"], Dk, z,
                                  a["h0"], a["dy"], a["dhf"], a["dx"], a["ddelta"], a["dA"], a["dBm"],
                                  a["dCm"], dD, dz, a["dh0"], ws, wsb, None)


# every case has exactly one defect, so no call reaches a launch
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(L=-1), 1), (dict(io=5), 1),
    (dict(N=24), 2), (dict(N=12), 2), (dict(N=512), 2), (dict(B=70000), 2),
    (dict(dy=None), 1), (dict(dA=None), 1), (dict(A=None), 1), (dict(dCm=None), 1), (dict(ddelta=None), 1),
    (dict(Dk=P), 1), (dict(dD=P), 1), (dict(z=P), 1), (dict(dz=P), 1),
    (dict(dh0=ctypes.c_void_p(0x10004)), 1), (dict(dy=ctypes.c_void_p(0x10002)), 1),
    (dict(ws=None, wsb=0), 3), (dict(wsb=64), 3),
])
def test_scan_bwd_rejects_bad_arguments(kw, status):
    assert _bwd(**kw) == status
    assert ops.lib().ssm_last_error().startswith(b"ssm_scan_bwd: ")


def test_scan_bwd_workspace_size():
    assert ssa.ssm_scan_bwd_workspace_size(1, 4096, 1536, 16) > 0
    assert ssa.ssm_scan_bwd_workspace_size(1, 0, 1536, 16) == 0
    assert ssa.ssm_scan_bwd_workspace_size(1, 4096, 1536, 32) > 0
    assert ssa.ssm_scan_bwd_workspace_size(1, 4096, 1536, 12) == 0  # unsupported N


def _scan_ex(disc=1, bias=None, sp=1, N=16, **kw):
    a = dict(B=1, L=64, D=64, io=1, x=P, delta=P, A=P, Bm=P, Cm=P, y=P)
    a.update(kw)
    return ops.lib().ssm_scan_fwd_ex(a["B"], a["L"], a["D"], N, a["io"], disc, bias, sp, a["x"], a["delta"],
                                     a["A"], a["Bm"], a["Cm"], None, None, None, a["y"], None, None, 0, None)


# one defect per case, so no call reaches a launch
@pytest.mark.parametrize("kw,status", [
    (dict(disc=2), 1), (dict(disc=-1), 1), (dict(N=12), 2),
    # N >= 64 is supported and needs a workspace, which these calls lack
    (dict(N=64), 3), (dict(N=256, disc=0, sp=1), 3),
    (dict(bias=ctypes.c_void_p(0x10004)), 1), (dict(x=None), 1), (dict(B=0), 1),
])
def test_scan_fwd_ex_rejects_bad_arguments(kw, status):
    assert _scan_ex(**kw) == status
    assert ops.lib().ssm_last_error().startswith(b"ssm_scan_fwd_ex: ")


def test_step_ex_rejects_bad_arguments():
    L = ops.lib()
    def call(disc=1, bias=None, N=16, state=P):
        return L.ssm_step_ex(2, 64, N, 1, disc, bias, 1, state, P, P, P, P, P, None, None, P, None)
    assert call(disc=3) == 1
    assert call(N=12) == 2
    assert call(state=None) == 1
    assert call(bias=ctypes.c_void_p(0x10008)) == 1
    assert ops.lib().ssm_last_error().startswith(b"ssm_step_ex: ")


def _noalloc(B=1, L=8, D=64, N=16, io=1, x=P, delta=P, A=P, Bm=P, Cm=P, Dk=None, z=None, h0=None, y=P, hf=None):
    return ops.lib().ssm_scan_fwd_noalloc(B, L, D, N, io, x, delta, A, Bm, Cm, Dk, z, h0, y, hf, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(L=-1), 1), (dict(io=5), 1), (dict(N=12), 2), (dict(x=None), 1),
    (dict(y=ctypes.c_void_p(0x10008)), 1),
    # fits ssm_scan_fwd with a workspace, but not the fixed scratch
    (dict(L=4096, D=1536, N=256), 2), (dict(B=2, L=8192, D=4096, N=32), 2),
])
def test_scan_fwd_noalloc_rejects_before_any_hip_call(kw, status):
    assert _noalloc(**kw) == status
    assert ops.lib().ssm_last_error().startswith(b"ssm_scan_fwd_noalloc: ")


def test_noalloc_scratch_limit_is_the_declared_one():
    src = open(HEADER).read()
    assert "#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in src
    limit = 128 << 20
    assert ssa.ssm_scan_workspace_size(8, 32768, 512, 16) <= limit      # the long-sequence workload fits
    assert ssa.ssm_scan_workspace_size(1, 4096, 1536, 256) > limit


def test_python_binding_has_every_entry_point_by_name():
    """The binding keeps the C names: every declared function except the library
    utilities (version, status strings, last error, timing hook) has a same-name
    Python function in the package."""
    utilities = {"ssm_abi_version", "ssm_last_error", "ssm_profile_events", "ssm_status_string"}
    missing = [n for n in declared_functions() if n not in utilities and not hasattr(ssa, n)]
    assert not missing, missing


def _scan3(B=1, L=8, D=64, N=16, io=1, x=P, delta=P, lam=P, Are=P, theta=P, Bm=P, Cm=P, Dk=None, z=None, h0=None,
           xp=None, bp=None, y=P, hf=None, ws=None, wsb=0):
    return ops.lib().ssm_scan3_fwd(B, L, D, N, io, x, delta, lam, Are, theta, Bm, Cm, Dk, z, h0, xp, bp, y, hf, ws,
                                   wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(L=-1), 1), (dict(io=3), 1), (dict(N=32), 2), (dict(N=12), 2), (dict(B=70000), 2),
    (dict(lam=None), 1), (dict(theta=None), 1), (dict(Are=None), 1), (dict(y=None), 1),
    (dict(xp=P), 1), (dict(bp=P), 1), (dict(h0=ctypes.c_void_p(0x10004)), 1),
    (dict(L=4096, D=1536), 3),
])
def test_scan3_rejects_bad_arguments(kw, status):
    assert _scan3(**kw) == status
    assert ops.lib().ssm_last_error().startswith(b"ssm_scan3_fwd: ")


def test_scan3_workspace_size():
    assert ssa.ssm_scan3_workspace_size(1, 4096, 1536, 16) > 0
    assert ssa.ssm_scan3_workspace_size(1, 32, 64, 16) == 0      # a single segment needs none
    assert ssa.ssm_scan3_workspace_size(1, 100, 64, 16) == 0     # one group of segments: one launch
    assert ssa.ssm_scan3_workspace_size(1, 4096, 1536, 32) == 0  # unsupported N


def _step3(B=2, D=64, N=16, io=1, state=P, x=P, delta=P, lam=P, Are=P, theta=P, Bm=P, Cm=P, Dk=None, z=None,
           xp=None, bp=None, y=P):
    return ops.lib().ssm_step3(B, D, N, io, state, x, delta, lam, Are, theta, Bm, Cm, Dk, z, xp, bp, y, None)


# one defect per case, so no call reaches a launch
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(D=0), 1), (dict(io=7), 1), (dict(N=12), 2), (dict(N=256), 2), (dict(B=70000), 2),
    (dict(D=1 << 26, N=64), 2), (dict(state=None), 1),
    (dict(lam=None), 1), (dict(theta=None), 1), (dict(y=None), 1), (dict(xp=P), 1), (dict(bp=P), 1),
    (dict(z=ctypes.c_void_p(0x10008)), 1),
])
def test_step3_rejects_bad_arguments(kw, status):
    assert _step3(**kw) == status
    assert ops.lib().ssm_last_error().startswith(b"ssm_step3: ")
