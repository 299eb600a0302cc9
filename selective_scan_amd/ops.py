"""ctypes marshalling for the C ABI of ``libssm_scan.so`` (see include/ssm_scan.h).

Argument checks here only concern the Python side (tensor device, dtype,
contiguity, shapes); the library validates again before any HIP call and every
non-OK status becomes an ``SsmError``.
"""
import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm_scan.so")

SSM_F32, SSM_BF16 = 0, 1
SSM_OK = 0

_lib = None


class SsmError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {detail}")


def lib():
    """The loaded ``libssm_scan.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m selective_scan_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, sz, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    L.ssm_abi_version.argtypes, L.ssm_abi_version.restype = [], i
    L.ssm_status_string.argtypes, L.ssm_status_string.restype = [i], ctypes.c_char_p
    L.ssm_last_error.argtypes, L.ssm_last_error.restype = [], ctypes.c_char_p
    L.ssm_scan_workspace_size.argtypes, L.ssm_scan_workspace_size.restype = [i, i, i, i], sz
    L.ssm_scan_fwd.argtypes = [i, i, i, i, i] + [vp] * 10 + [vp, sz, vp]
    L.ssm_scan_fwd.restype = i
    L.ssm_scan_fwd_noalloc.argtypes = [i, i, i, i, i] + [vp] * 10 + [vp]
    L.ssm_scan_fwd_noalloc.restype = i
    L.ssm_scan3_workspace_size.argtypes, L.ssm_scan3_workspace_size.restype = [i, i, i, i], sz
    L.ssm_scan3_fwd.argtypes = [i, i, i, i, i] + [vp] * 14 + [vp, sz, vp]
    L.ssm_scan3_fwd.restype = i
    L.ssm_scan_fwd_ex.argtypes = [i, i, i, i, i, i, vp, i] + [vp] * 10 + [vp, sz, vp]
    L.ssm_scan_fwd_ex.restype = i
    L.ssm_step_ex.argtypes = [i, i, i, i, i, vp, i] + [fp] + [vp] * 8 + [vp]
    L.ssm_step_ex.restype = i
    L.ssm_scan_bwd_workspace_size.argtypes, L.ssm_scan_bwd_workspace_size.restype = [i, i, i, i], sz
    L.ssm_scan_bwd.argtypes = [i, i, i, i, i] + [vp] * 18 + [vp, sz, vp]
    L.ssm_scan_bwd.restype = i
    L.ssm_ssd_workspace_size.argtypes, L.ssm_ssd_workspace_size.restype = [i] * 6, sz
    L.ssm_ssd_fwd.argtypes = [i] * 7 + [vp] * 10 + [vp, sz, vp]
    L.ssm_ssd_fwd.restype = i
    L.ssm_step.argtypes = [i, i, i, i] + [fp] + [vp] * 8 + [vp]
    L.ssm_step.restype = i
    L.ssm_ssd_step.argtypes = [i, i, i, i, i] + [fp] + [vp] * 8 + [vp]
    L.ssm_ssd_step.restype = i
    L.ssm_step3.argtypes = [i, i, i, i] + [fp] + [vp] * 12 + [vp]
    L.ssm_step3.restype = i
    L.ssm_diag_valu_rate.argtypes, L.ssm_diag_valu_rate.restype = [i, i, i, vp, vp], i
    L.ssm_diag_stream_scale.argtypes, L.ssm_diag_stream_scale.restype = [vp, sz, ctypes.c_float, vp], i
    L.ssm_diag_copy.argtypes, L.ssm_diag_copy.restype = [vp, vp, sz, vp], i
    _lib = L
    return _lib


# ------------------------------------------------------------------ helpers
def _io_code(t):
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    if t.dtype == torch.float32:
        return SSM_F32
    raise TypeError(f"io tensors must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Allocation context for a call launched on ``stream``: tensors this binding
    allocates (outputs, workspace) are taken from the caching allocator on the
    launch stream itself, so a block freed on return (the workspace) is only handed
    out again to work queued after these kernels on that stream."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _raise(fn, status):
    L = lib()
    raise SsmError(fn, status, L.ssm_last_error().decode())


# ------------------------------------------------------------------ Mamba-1
def ssm_scan_workspace_size(B, L, D, N):
    return int(lib().ssm_scan_workspace_size(B, L, D, N))


SSM_DISC = {"euler": 0, "zoh": 1}


def ssm_scan_fwd(x, delta, A, Bm, Cm, D=None, z=None, h0=None, *, y=None, h_final=None,
                 workspace=None, stream=None, want_final_state=True):
    """Mamba-1 selective scan. x, delta, z: [B, L, D]; Bm, Cm: [B, L, N] (bf16 or fp32);
    A: [D, N], D: [D], h0: [B, D, N] fp32. Returns (y, h_final) (h_final None if not wanted)."""
    return _scan_fwd("ssm_scan_fwd", x, delta, A, Bm, Cm, D, z, h0, y, h_final, workspace, stream,
                     want_final_state, None)


def ssm_scan_fwd_noalloc(x, delta, A, Bm, Cm, D=None, z=None, h0=None, *, y, h_final=None, stream=None):
    """``ssm_scan_fwd`` on the library's fixed per-GPU scratch (no workspace, no
    allocation here or in the library): the caller passes every output tensor.
    Calls that may overlap on one GPU race on the shared scratch."""
    Bb, L, Dd = x.shape
    N = A.shape[1]
    dev, io = x.device, x.dtype
    for t, nm, shp, dt, req in ((x, "x", (Bb, L, Dd), io, True), (delta, "delta", (Bb, L, Dd), io, True),
                                (A, "A", (Dd, N), torch.float32, True), (Bm, "Bm", (Bb, L, N), io, True),
                                (Cm, "Cm", (Bb, L, N), io, True), (D, "D", (Dd,), torch.float32, False),
                                (z, "z", (Bb, L, Dd), io, False), (h0, "h0", (Bb, Dd, N), torch.float32, False),
                                (y, "y", (Bb, L, Dd), io, True),
                                (h_final, "h_final", (Bb, Dd, N), torch.float32, False)):
        _check(t, nm, shp, dt, dev, required=req)
    st = lib().ssm_scan_fwd_noalloc(Bb, L, Dd, N, _io_code(x), _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                                    _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_final), _stream(dev, stream))
    if st != SSM_OK:
        _raise("ssm_scan_fwd_noalloc", st)
    return y, h_final


def ssm_scan_fwd_ex(x, delta, A, Bm, Cm, D=None, z=None, h0=None, *, disc="euler", delta_bias=None,
                    delta_softplus=False, y=None, h_final=None, workspace=None, stream=None,
                    want_final_state=True):
    """``ssm_scan_fwd`` with disc = "euler" | "zoh" (exact zero-order hold) and
    Delta = [softplus](delta + delta_bias) inside the kernels (delta_bias: [D] fp32)."""
    return _scan_fwd("ssm_scan_fwd_ex", x, delta, A, Bm, Cm, D, z, h0, y, h_final, workspace, stream,
                     want_final_state, (SSM_DISC[disc], delta_bias, bool(delta_softplus)))


def _scan_fwd(fn, x, delta, A, Bm, Cm, D, z, h0, y, h_final, workspace, stream, want_final_state, ex):
    Bb, L, Dd = x.shape
    N = A.shape[1]
    dev, io = x.device, x.dtype
    _check(delta, "delta", (Bb, L, Dd), io, dev)
    _check(A, "A", (Dd, N), torch.float32, dev)
    _check(Bm, "Bm", (Bb, L, N), io, dev)
    _check(Cm, "Cm", (Bb, L, N), io, dev)
    _check(D, "D", (Dd,), torch.float32, dev, required=False)
    _check(z, "z", (Bb, L, Dd), io, dev, required=False)
    _check(h0, "h0", (Bb, Dd, N), torch.float32, dev, required=False)
    _check(x, "x", (Bb, L, Dd), io, dev)
    need = ssm_scan_workspace_size(Bb, L, Dd, N)
    with _on(stream):
        if y is None:
            y = torch.empty((Bb, L, Dd), dtype=io, device=dev)
        if want_final_state and h_final is None:
            h_final = torch.empty((Bb, Dd, N), dtype=torch.float32, device=dev)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(y, "y", (Bb, L, Dd), io, dev)
    _check(h_final, "h_final", (Bb, Dd, N), torch.float32, dev, required=False)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z), _ptr(h0), _ptr(y),
            _ptr(h_final), _ptr(workspace), wbytes, _stream(dev, stream))
    if ex is None:
        st = lib().ssm_scan_fwd(Bb, L, Dd, N, _io_code(x), *args)
    else:
        disc, bias, sp = ex
        _check(bias, "delta_bias", (Dd,), torch.float32, dev, required=False)
        st = lib().ssm_scan_fwd_ex(Bb, L, Dd, N, _io_code(x), disc, _ptr(bias), int(sp), *args)
    if st != SSM_OK:
        _raise(fn, st)
    return y, h_final


def ssm_scan3_workspace_size(B, L, D, N):
    return int(lib().ssm_scan3_workspace_size(B, L, D, N))


def ssm_scan3_fwd(x, delta, lam, Are, theta, Bm, Cm, D=None, z=None, h0=None, x_prev=None, B_prev=None, *,
                  y=None, h_final=None, workspace=None, stream=None, want_final_state=True):
    """Mamba-3 scan. x, delta, lam, z: [B, L, D]; Bm, Cm: [B, L, N] (bf16 or fp32); Are,
    theta: [D, N] fp32; D: [D]; h0: [B, D, N, 2] fp32 (real, imaginary); x_prev [B, D] and
    B_prev [B, N]: the token before the sequence. Returns (y, h_final [B, D, N, 2])."""
    Bb, L, Dd = x.shape
    N = Are.shape[1]
    dev, io = x.device, x.dtype
    for t, nm, shp, dt, req in ((x, "x", (Bb, L, Dd), io, True), (delta, "delta", (Bb, L, Dd), io, True),
                                (lam, "lam", (Bb, L, Dd), io, True), (Are, "Are", (Dd, N), torch.float32, True),
                                (theta, "theta", (Dd, N), torch.float32, True), (Bm, "Bm", (Bb, L, N), io, True),
                                (Cm, "Cm", (Bb, L, N), io, True), (D, "D", (Dd,), torch.float32, False),
                                (z, "z", (Bb, L, Dd), io, False), (h0, "h0", (Bb, Dd, N, 2), torch.float32, False),
                                (x_prev, "x_prev", (Bb, Dd), io, False), (B_prev, "B_prev", (Bb, N), io, False)):
        _check(t, nm, shp, dt, dev, required=req)
    need = ssm_scan3_workspace_size(Bb, L, Dd, N)
    with _on(stream):
        if y is None:
            y = torch.empty((Bb, L, Dd), dtype=io, device=dev)
        if want_final_state and h_final is None:
            h_final = torch.empty((Bb, Dd, N, 2), dtype=torch.float32, device=dev)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(y, "y", (Bb, L, Dd), io, dev)
    _check(h_final, "h_final", (Bb, Dd, N, 2), torch.float32, dev, required=False)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ssm_scan3_fwd(Bb, L, Dd, N, _io_code(x), _ptr(x), _ptr(delta), _ptr(lam), _ptr(Are), _ptr(theta),
                             _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z), _ptr(h0), _ptr(x_prev), _ptr(B_prev), _ptr(y),
                             _ptr(h_final), _ptr(workspace), wbytes, _stream(dev, stream))
    if st != SSM_OK:
        _raise("ssm_scan3_fwd", st)
    return y, h_final


def ssm_scan_bwd_workspace_size(B, L, D, N):
    return int(lib().ssm_scan_bwd_workspace_size(B, L, D, N))


def ssm_scan_bwd(x, delta, A, Bm, Cm, dy, D=None, z=None, h0=None, dh_final=None, *,
                 want_dh0=True, out=None, workspace=None, stream=None):
    """Gradient of ``ssm_scan_fwd`` for l = sum(dy * y) + sum(dh_final * h_final).

    Inputs as for ``ssm_scan_fwd``; dy: [B, L, D] io dtype; dh_final: [B, D, N] fp32
    or None. Returns a dict with dx, ddelta [B, L, D]; dA [D, N] fp32; dBm, dCm
    [B, L, N]; dD [D] fp32 (None without D); dz [B, L, D] (None without z); dh0
    [B, D, N] fp32 (None unless want_dh0). ``out`` may supply any of these tensors."""
    Bb, L, Dd = x.shape
    N = A.shape[1]
    dev, io = x.device, x.dtype
    _check(x, "x", (Bb, L, Dd), io, dev)
    _check(delta, "delta", (Bb, L, Dd), io, dev)
    _check(A, "A", (Dd, N), torch.float32, dev)
    _check(Bm, "Bm", (Bb, L, N), io, dev)
    _check(Cm, "Cm", (Bb, L, N), io, dev)
    _check(dy, "dy", (Bb, L, Dd), io, dev)
    _check(D, "D", (Dd,), torch.float32, dev, required=False)
    _check(z, "z", (Bb, L, Dd), io, dev, required=False)
    _check(h0, "h0", (Bb, Dd, N), torch.float32, dev, required=False)
    _check(dh_final, "dh_final", (Bb, Dd, N), torch.float32, dev, required=False)
    shapes = dict(dx=((Bb, L, Dd), io), ddelta=((Bb, L, Dd), io), dA=((Dd, N), torch.float32),
                  dBm=((Bb, L, N), io), dCm=((Bb, L, N), io), dD=((Dd,), torch.float32),
                  dz=((Bb, L, Dd), io), dh0=((Bb, Dd, N), torch.float32))
    wanted = dict(dD=D is not None, dz=z is not None, dh0=want_dh0)
    g = dict(out or {})
    need = ssm_scan_bwd_workspace_size(Bb, L, Dd, N)
    with _on(stream):
        for k, (shp, dt) in shapes.items():
            if not wanted.get(k, True):
                g[k] = None
                continue
            if g.get(k) is None:
                g[k] = torch.empty(shp, dtype=dt, device=dev)
            _check(g[k], k, shp, dt, dev)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ssm_scan_bwd(Bb, L, Dd, N, _io_code(x), _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm),
                            _ptr(Cm), _ptr(D), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dh_final),
                            *(_ptr(g[k]) for k in ("dx", "ddelta", "dA", "dBm", "dCm", "dD", "dz", "dh0")),
                            _ptr(workspace), wbytes, _stream(dev, stream))
    if st != SSM_OK:
        _raise("ssm_scan_bwd", st)
    return g


# ------------------------------------------------------------------ SSD
def ssm_ssd_workspace_size(B, L, H, P, N, chunk=0):
    return int(lib().ssm_ssd_workspace_size(B, L, H, P, N, chunk))


def ssm_ssd_fwd(x, delta, A, Bm, Cm, D=None, z=None, h0=None, *, chunk=0, y=None,
                h_final=None, workspace=None, stream=None, want_final_state=True):
    """Mamba-2 SSD chunked scan. x, z: [B, L, H, P]; delta: [B, L, H]; Bm, Cm: [B, L, N];
    A, D: [H] fp32; h0: [B, H, N, P] fp32. Returns (y, h_final)."""
    Bb, L, H, P = x.shape
    N = Bm.shape[2]
    dev, io = x.device, x.dtype
    _check(x, "x", (Bb, L, H, P), io, dev)
    _check(delta, "delta", (Bb, L, H), io, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(Bm, "Bm", (Bb, L, N), io, dev)
    _check(Cm, "Cm", (Bb, L, N), io, dev)
    _check(D, "D", (H,), torch.float32, dev, required=False)
    _check(z, "z", (Bb, L, H, P), io, dev, required=False)
    _check(h0, "h0", (Bb, H, N, P), torch.float32, dev, required=False)
    need = ssm_ssd_workspace_size(Bb, L, H, P, N, chunk)
    with _on(stream):
        if y is None:
            y = torch.empty((Bb, L, H, P), dtype=io, device=dev)
        if want_final_state and h_final is None:
            h_final = torch.empty((Bb, H, N, P), dtype=torch.float32, device=dev)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(y, "y", (Bb, L, H, P), io, dev)
    _check(h_final, "h_final", (Bb, H, N, P), torch.float32, dev, required=False)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ssm_ssd_fwd(Bb, L, H, P, N, int(chunk), _io_code(x), _ptr(x), _ptr(delta), _ptr(A),
                           _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_final),
                           _ptr(workspace), wbytes, _stream(dev, stream))
    if st != SSM_OK:
        _raise("ssm_ssd_fwd", st)
    return y, h_final


# ------------------------------------------------------------------ decode
def ssm_step(state, x, delta, A, Bm, Cm, D=None, z=None, *, y=None, stream=None):
    """One decode step. state: [B, D, N] fp32 (updated in place); x, delta, z: [B, D];
    Bm, Cm: [B, N]; A: [D, N]; D: [D]. Returns y [B, D]."""
    return _step("ssm_step", state, x, delta, A, Bm, Cm, D, z, y, stream, None)


def ssm_step_ex(state, x, delta, A, Bm, Cm, D=None, z=None, *, disc="euler", delta_bias=None,
                delta_softplus=False, y=None, stream=None):
    """``ssm_step`` with the options of ``ssm_scan_fwd_ex``."""
    return _step("ssm_step_ex", state, x, delta, A, Bm, Cm, D, z, y, stream,
                 (SSM_DISC[disc], delta_bias, bool(delta_softplus)))


def _step(fn, state, x, delta, A, Bm, Cm, D, z, y, stream, ex):
    Bb, Dd, N = state.shape
    dev, io = x.device, x.dtype
    _check(state, "state", (Bb, Dd, N), torch.float32, dev)
    _check(x, "x", (Bb, Dd), io, dev)
    _check(delta, "delta", (Bb, Dd), io, dev)
    _check(A, "A", (Dd, N), torch.float32, dev)
    _check(Bm, "Bm", (Bb, N), io, dev)
    _check(Cm, "Cm", (Bb, N), io, dev)
    _check(D, "D", (Dd,), torch.float32, dev, required=False)
    _check(z, "z", (Bb, Dd), io, dev, required=False)
    if y is None:
        with _on(stream):
            y = torch.empty((Bb, Dd), dtype=io, device=dev)
    _check(y, "y", (Bb, Dd), io, dev)
    args = (_ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z), _ptr(y),
            _stream(dev, stream))
    if ex is None:
        st = lib().ssm_step(Bb, Dd, N, _io_code(x), *args)
    else:
        disc, bias, sp = ex
        _check(bias, "delta_bias", (Dd,), torch.float32, dev, required=False)
        st = lib().ssm_step_ex(Bb, Dd, N, _io_code(x), disc, _ptr(bias), int(sp), *args)
    if st != SSM_OK:
        _raise(fn, st)
    return y


def ssm_ssd_step(state, x, delta, A, Bm, Cm, D=None, z=None, *, y=None, stream=None):
    """One Mamba-2 decode step. state: [B, H, N, P] fp32 (updated in place); x, z: [B, H, P];
    delta: [B, H]; Bm, Cm: [B, N]; A: [H]; D: [H]. Returns y [B, H, P]."""
    Bb, H, N, P = state.shape
    dev, io = x.device, x.dtype
    _check(state, "state", (Bb, H, N, P), torch.float32, dev)
    _check(x, "x", (Bb, H, P), io, dev)
    _check(delta, "delta", (Bb, H), io, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(Bm, "Bm", (Bb, N), io, dev)
    _check(Cm, "Cm", (Bb, N), io, dev)
    _check(D, "D", (H,), torch.float32, dev, required=False)
    _check(z, "z", (Bb, H, P), io, dev, required=False)
    if y is None:
        with _on(stream):
            y = torch.empty((Bb, H, P), dtype=io, device=dev)
    _check(y, "y", (Bb, H, P), io, dev)
    st = lib().ssm_ssd_step(Bb, H, P, N, _io_code(x), _ptr(state), _ptr(x), _ptr(delta), _ptr(A),
                            _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z), _ptr(y), _stream(dev, stream))
    if st != SSM_OK:
        _raise("ssm_ssd_step", st)
    return y


def ssm_step3(state, x, delta, lam, Are, theta, Bm, Cm, D=None, z=None, x_prev=None, B_prev=None, *, y=None,
              stream=None):
    """One Mamba-3 decode step. state: [B, D, N, 2] fp32 (real, imaginary; updated in
    place); x, delta, lam, z: [B, D]; Bm, Cm: [B, N]; Are, theta: [D, N] fp32; D: [D];
    x_prev [B, D] and B_prev [B, N]: the previous token. Returns y [B, D]."""
    Bb, Dd, N, two = state.shape
    dev, io = x.device, x.dtype
    _check(state, "state", (Bb, Dd, N, 2), torch.float32, dev)
    for t, nm, shp, dt, req in ((x, "x", (Bb, Dd), io, True), (delta, "delta", (Bb, Dd), io, True),
                                (lam, "lam", (Bb, Dd), io, True), (Are, "Are", (Dd, N), torch.float32, True),
                                (theta, "theta", (Dd, N), torch.float32, True), (Bm, "Bm", (Bb, N), io, True),
                                (Cm, "Cm", (Bb, N), io, True), (D, "D", (Dd,), torch.float32, False),
                                (z, "z", (Bb, Dd), io, False), (x_prev, "x_prev", (Bb, Dd), io, False),
                                (B_prev, "B_prev", (Bb, N), io, False)):
        _check(t, nm, shp, dt, dev, required=req)
    if y is None:
        with _on(stream):
            y = torch.empty((Bb, Dd), dtype=io, device=dev)
    _check(y, "y", (Bb, Dd), io, dev)
    st = lib().ssm_step3(Bb, Dd, N, _io_code(x), _ptr(state), _ptr(x), _ptr(delta), _ptr(lam), _ptr(Are),
                         _ptr(theta), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z), _ptr(x_prev), _ptr(B_prev), _ptr(y),
                         _stream(dev, stream))
    if st != SSM_OK:
        _raise("ssm_step3", st)
    return y


# ------------------------------------------------------------------ diagnostics
def ssm_diag_valu_rate(mode, out, iters, stream=None):
    """VALU issue-rate probe (mode 0 exp, 1 fma, 2 exp:fma 1:3, 3 sin, 4 cos); ``out`` is an fp32
    tensor of blocks * 256 elements. Returns the number of ops it issues."""
    blocks = out.numel() // 256
    st = lib().ssm_diag_valu_rate(int(mode), blocks, int(iters), _ptr(out), _stream(out.device, stream))
    if st != SSM_OK:
        _raise("ssm_diag_valu_rate", st)
    return blocks * 256 * 32 * int(iters)


def ssm_diag_stream_scale(t, s, stream=None):
    """t *= s in place on a contiguous fp32 tensor (the pure-streaming floor)."""
    _check(t, "t", tuple(t.shape), torch.float32, t.device)
    st = lib().ssm_diag_stream_scale(_ptr(t), t.numel(), float(s), _stream(t.device, stream))
    if st != SSM_OK:
        _raise("ssm_diag_stream_scale", st)


def ssm_diag_copy(src, dst, stream=None):
    """dst = src for contiguous fp32 tensors of the same shape (the copy kernel the HBM
    byte counters are calibrated with)."""
    _check(src, "src", tuple(src.shape), torch.float32, src.device)
    _check(dst, "dst", tuple(src.shape), torch.float32, src.device)
    st = lib().ssm_diag_copy(_ptr(src), _ptr(dst), src.numel(), _stream(src.device, stream))
    if st != SSM_OK:
        _raise("ssm_diag_copy", st)
