"""Helpers for the GPU parity tests: move stored inputs to the device, read
results back as exact float64, and call the oracle on the same stored bits."""
import numpy as np
import torch

import oracle
import ssm_inputs as si

DEV = "cuda:0"


def to_dev(w, keys):
    return {k: (si.to_torch(w[k], DEV) if w.get(k) is not None else None) for k in keys}


def out_f64(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return si.to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def storage(w):
    return "bf16" if w["dtype"] == si.BF16 else "f32"


def oracle_scan(w, sel=None):
    """fp64 oracle on the stored inputs, optionally on a subset ``sel`` of channels."""
    f = {k: si.to_f64(w[k]) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    if sel is not None:
        for k in ("x", "delta", "z"):
            if f[k] is not None:
                f[k] = np.ascontiguousarray(f[k][:, :, sel])
        f["A"] = np.ascontiguousarray(f["A"][sel])
        if f["D"] is not None:
            f["D"] = np.ascontiguousarray(f["D"][sel])
        if f["h0"] is not None:
            f["h0"] = np.ascontiguousarray(f["h0"][:, sel])
    return oracle.scan(f["x"], f["delta"], f["A"], f["Bm"], f["Cm"], D=f["D"], z=f["z"], h0=f["h0"])


def gpu_scan(w, **kw):
    import selective_scan_amd as ssa
    t = to_dev(w, ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0"))
    y, hf = ssa.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"],
                             h0=t["h0"], **kw)
    torch.cuda.synchronize()
    return y, hf


def oracle_scan_bwd(w, gw, sel=None):
    """fp64 oracle gradients on the stored inputs and cotangents. With ``sel`` the
    per-channel outputs are computed for those channels only (dBm, dCm are then
    partial sums and must not be compared)."""
    f = {k: si.to_f64(w[k]) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0")}
    dy, dhf = si.to_f64(gw["dy"]), si.to_f64(gw["dh_final"])
    if sel is not None:
        for k in ("x", "delta", "z"):
            if f[k] is not None:
                f[k] = np.ascontiguousarray(f[k][:, :, sel])
        dy = np.ascontiguousarray(dy[:, :, sel])
        f["A"] = np.ascontiguousarray(f["A"][sel])
        if f["D"] is not None:
            f["D"] = np.ascontiguousarray(f["D"][sel])
        for k in ("h0",):
            if f[k] is not None:
                f[k] = np.ascontiguousarray(f[k][:, sel])
        if dhf is not None:
            dhf = np.ascontiguousarray(dhf[:, sel])
    return oracle.scan_bwd(f["x"], f["delta"], f["A"], f["Bm"], f["Cm"], dy, D=f["D"], z=f["z"],
                           h0=f["h0"], dh_final=dhf)


def gpu_scan_bwd(w, gw, **kw):
    import selective_scan_amd as ssa
    t = to_dev(w, ("x", "delta", "z", "Bm", "Cm", "A", "D", "h0"))
    g = to_dev(gw, ("dy", "dh_final"))
    out = ssa.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], g["dy"], D=t["D"], z=t["z"],
                           h0=t["h0"], dh_final=g["dh_final"], **kw)
    torch.cuda.synchronize()
    return out
