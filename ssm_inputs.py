"""Seeded synthetic inputs for the selective-scan workloads.

This module is shared by the tests, the benchmark and the smoke check. It holds
no part of the scan's arithmetic: it only draws random numbers, shapes them like
the workloads below and rounds them ONCE (round-to-nearest-even) from float64 to
the storage dtype. The oracle and the GPU path consume the same stored bits.

Distributions (the same for every workload unless stated):
  x, z          ~ N(0, 1)
  B, C          ~ N(0, 1) / sqrt(N), one group shared by all channels / heads
  dt            = exp(U[ln 1e-3, ln 1e-1]), drawn once per channel (per head for SSD)
  Delta[.., c]  = softplus(0.5 * eps + ln(expm1(dt_c))), eps ~ N(0, 1) per element
  A (Mamba-1)   A[d, n] = -(n + 1)                         (fp32)
  A (SSD)       A_h = -exp(U[ln 1, ln 16])                 (fp32)
  D             ~ N(0, 1)                                  (fp32)
  state0        ~ 0.1 * N(0, 1)                            (fp32, decode only)
  dy            ~ N(0, 1)            (gradient of y, backward pass)
  dh_final      ~ 0.1 * N(0, 1)      (fp32, gradient of the final state, backward pass)
Random streams: ``numpy.random.default_rng([seed, tensor_id])`` (PCG64) with a
fixed id per tensor, so every tensor is reproducible on its own.
"""
import math

import numpy as np

# fixed stream ids, one per tensor
TID_DT, TID_X, TID_Z, TID_EPS, TID_B, TID_C, TID_D, TID_A, TID_STATE0, TID_DY, TID_DHF = range(11)
TID_LAM, TID_THETA, TID_PREV = 11, 12, 13

BF16, F32 = "bf16", "f32"


# ----------------------------------------------------------------- rounding
def round_bf16_bits(v):
    """float64 -> bfloat16 bit patterns (np.uint16), one RNE rounding step.

    Works on the float64 bit pattern: keep sign, exponent and the top 7 stored
    mantissa bits, rounding the dropped 45 bits to nearest-even. Values must be
    zero or normal in bfloat16's range (true for every workload here).
    """
    v = np.ascontiguousarray(v, dtype=np.float64)
    a = np.abs(v)
    nz = a != 0
    if np.any(~np.isfinite(v)) or np.any(a[nz] < 2.0 ** -126) or np.any(a >= 3.3e38):
        raise ValueError("value outside bf16 normal range")
    u = v.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + (np.uint64((1 << 44) - 1) + lsb)) & ~np.uint64((1 << 45) - 1)
    f32 = r.view(np.float64).astype(np.float32)  # exact: 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def store(v, dtype):
    """Round float64 values to the storage dtype: uint16 bf16 bits or float32."""
    if dtype == BF16:
        return round_bf16_bits(v)
    if dtype == F32:
        return np.asarray(v, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def to_f64(a):
    """Exact float64 value of a stored array (bf16 bits, float32 or float64)."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def to_torch(a, device="cpu"):
    """Stored numpy array -> torch tensor (bf16 bits become torch.bfloat16)."""
    import torch
    if a is None:
        return None
    a = np.require(a, requirements=["C", "W"])
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


# ----------------------------------------------------------------- draws
def _rng(seed, tid):
    return np.random.default_rng([int(seed), int(tid)])


def _normal(seed, tid, shape):
    return _rng(seed, tid).standard_normal(shape)


def _dt_per_channel(seed, n):
    u = _rng(seed, TID_DT).uniform(math.log(1e-3), math.log(1e-1), size=n)
    return np.exp(u)


def _delta(seed, shape, dt_c):
    """softplus(0.5 eps + ln(expm1(dt_c))) with dt_c broadcast over the last axis."""
    eps = _normal(seed, TID_EPS, shape)
    pre = 0.5 * eps + np.log(np.expm1(dt_c))
    return np.logaddexp(0.0, pre)


# ----------------------------------------------------------------- workloads
def scan_inputs(B, L, D, N, dtype=BF16, seed=0, with_D=True, with_z=True, with_h0=False):
    """Mamba-1 scan inputs. x, delta, z [B,L,D]; Bm, Cm [B,L,N] in ``dtype``;
    A [D,N], D [D], h0 [B,D,N] in float32."""
    out = {}
    out["x"] = store(_normal(seed, TID_X, (B, L, D)), dtype)
    out["delta"] = store(_delta(seed, (B, L, D), _dt_per_channel(seed, D)), dtype)
    out["z"] = store(_normal(seed, TID_Z, (B, L, D)), dtype) if with_z else None
    s = 1.0 / math.sqrt(N)
    out["Bm"] = store(_normal(seed, TID_B, (B, L, N)) * s, dtype)
    out["Cm"] = store(_normal(seed, TID_C, (B, L, N)) * s, dtype)
    out["A"] = np.ascontiguousarray(np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (D, N)))
    out["D"] = _normal(seed, TID_D, (D,)).astype(np.float32) if with_D else None
    out["h0"] = (0.1 * _normal(seed, TID_STATE0, (B, D, N))).astype(np.float32) if with_h0 else None
    out["dtype"] = dtype
    return out


def scan3_inputs(B, L, D, N, dtype=BF16, seed=0, with_D=True, with_z=True, with_h0=False, with_prev=False):
    """Mamba-3 scan inputs: those of ``scan_inputs`` (A as the real part Are) plus
    lam = sigmoid(N(0,1)) [B,L,D] in ``dtype``, rotation rates theta ~ U(-pi, pi) [D,N]
    float32, complex h0 [B,D,N,2] (real, imaginary) float32 and the token before the
    sequence, x_prev [B,D] and B_prev [B,N] in ``dtype``."""
    out = scan_inputs(B, L, D, N, dtype=dtype, seed=seed, with_D=with_D, with_z=with_z, with_h0=False)
    out["Are"] = out.pop("A")
    out["lam"] = store(1.0 / (1.0 + np.exp(-_normal(seed, TID_LAM, (B, L, D)))), dtype)
    out["theta"] = _rng(seed, TID_THETA).uniform(-math.pi, math.pi, (D, N)).astype(np.float32)
    out["h0"] = (0.1 * _normal(seed, TID_STATE0, (B, D, N, 2))).astype(np.float32) if with_h0 else None
    if with_prev:
        r = _rng(seed, TID_PREV)
        out["x_prev"] = store(r.standard_normal((B, D)), dtype)
        out["B_prev"] = store(r.standard_normal((B, N)) / math.sqrt(N), dtype)
    else:
        out["x_prev"] = out["B_prev"] = None
    return out


def scan_raw_delta(B, L, D, dtype=BF16, seed=0):
    """Delta before its softplus, for the kernels that apply softplus(delta + bias)
    themselves: delta = 0.5 eps [B,L,D] in ``dtype`` and delta_bias = ln(expm1(dt_c))
    [D] float32, so softplus(delta + delta_bias) has the distribution of ``scan_inputs``'
    Delta (the same eps and dt_c streams)."""
    eps = _normal(seed, TID_EPS, (B, L, D))
    return dict(delta=store(0.5 * eps, dtype),
                delta_bias=np.log(np.expm1(_dt_per_channel(seed, D))).astype(np.float32))


def scan_grad_inputs(B, L, D, N, dtype=BF16, seed=0, with_dh_final=True):
    """Cotangents for the backward pass of the Mamba-1 scan: dy [B,L,D] in
    ``dtype`` and dh_final [B,D,N] in float32 (None when not wanted)."""
    return dict(dy=store(_normal(seed, TID_DY, (B, L, D)), dtype),
                dh_final=(0.1 * _normal(seed, TID_DHF, (B, D, N))).astype(np.float32) if with_dh_final else None)


def ssd_inputs(B, L, H, P, N, dtype=BF16, seed=0, with_D=False, with_z=False, with_h0=False):
    """SSD inputs. x, z [B,L,H,P]; delta [B,L,H]; Bm, Cm [B,L,N] in ``dtype``;
    A [H], D [H], h0 [B,H,N,P] in float32."""
    out = {}
    out["x"] = store(_normal(seed, TID_X, (B, L, H, P)), dtype)
    out["delta"] = store(_delta(seed, (B, L, H), _dt_per_channel(seed, H)), dtype)
    out["z"] = store(_normal(seed, TID_Z, (B, L, H, P)), dtype) if with_z else None
    s = 1.0 / math.sqrt(N)
    out["Bm"] = store(_normal(seed, TID_B, (B, L, N)) * s, dtype)
    out["Cm"] = store(_normal(seed, TID_C, (B, L, N)) * s, dtype)
    out["A"] = (-np.exp(_rng(seed, TID_A).uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    out["D"] = _normal(seed, TID_D, (H,)).astype(np.float32) if with_D else None
    out["h0"] = (0.1 * _normal(seed, TID_STATE0, (B, H, N, P))).astype(np.float32) if with_h0 else None
    out["dtype"] = dtype
    return out


def step_inputs(B, D, N, steps, dtype=BF16, seed=0, with_D=True, with_z=True):
    """Decode inputs: state0 [B,D,N] fp32 ~ 0.1 N(0,1); per-token x, delta, z
    [steps,B,D] and Bm, Cm [steps,B,N] in ``dtype``; A [D,N], D [D] fp32."""
    out = {}
    out["state0"] = (0.1 * _normal(seed, TID_STATE0, (B, D, N))).astype(np.float32)
    out["x"] = store(_normal(seed, TID_X, (steps, B, D)), dtype)
    out["delta"] = store(_delta(seed, (steps, B, D), _dt_per_channel(seed, D)), dtype)
    out["z"] = store(_normal(seed, TID_Z, (steps, B, D)), dtype) if with_z else None
    s = 1.0 / math.sqrt(N)
    out["Bm"] = store(_normal(seed, TID_B, (steps, B, N)) * s, dtype)
    out["Cm"] = store(_normal(seed, TID_C, (steps, B, N)) * s, dtype)
    out["A"] = np.ascontiguousarray(np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (D, N)))
    out["D"] = _normal(seed, TID_D, (D,)).astype(np.float32) if with_D else None
    out["dtype"] = dtype
    return out


def ssd_step_inputs(B, H, P, N, steps, dtype=BF16, seed=0, with_D=True, with_z=True):
    """Mamba-2 decode inputs: state0 [B,H,N,P] fp32 ~ 0.1 N(0,1); per-token x, z
    [steps,B,H,P], delta [steps,B,H] and Bm, Cm [steps,B,N] in ``dtype``; A [H],
    D [H] fp32 (distributions as ``ssd_inputs``)."""
    out = {}
    out["state0"] = (0.1 * _normal(seed, TID_STATE0, (B, H, N, P))).astype(np.float32)
    out["x"] = store(_normal(seed, TID_X, (steps, B, H, P)), dtype)
    out["delta"] = store(_delta(seed, (steps, B, H), _dt_per_channel(seed, H)), dtype)
    out["z"] = store(_normal(seed, TID_Z, (steps, B, H, P)), dtype) if with_z else None
    s = 1.0 / math.sqrt(N)
    out["Bm"] = store(_normal(seed, TID_B, (steps, B, N)) * s, dtype)
    out["Cm"] = store(_normal(seed, TID_C, (steps, B, N)) * s, dtype)
    out["A"] = (-np.exp(_rng(seed, TID_A).uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    out["D"] = _normal(seed, TID_D, (H,)).astype(np.float32) if with_D else None
    out["dtype"] = dtype
    return out


# Workloads of the benchmark configurations (sizes of the pages' workloads).
WORKLOADS = {
    "scan_f32_B1_L256_D64_N16": dict(kind="scan", B=1, L=256, D=64, N=16, dtype=F32),
    "scan_bf16_B1_L4096_D1536_N16": dict(kind="scan", B=1, L=4096, D=1536, N=16, dtype=BF16),
    "scan_bf16_B8_L32768_D512_N16": dict(kind="scan", B=8, L=32768, D=512, N=16, dtype=BF16),
    # ssm-bench's state-dimension sweep at the headline layer's size
    "scan_bf16_B1_L4096_D1536_N64": dict(kind="scan", B=1, L=4096, D=1536, N=64, dtype=BF16),
    "scan_bf16_B1_L4096_D1536_N128": dict(kind="scan", B=1, L=4096, D=1536, N=128, dtype=BF16),
    "scan_bf16_B1_L4096_D1536_N256": dict(kind="scan", B=1, L=4096, D=1536, N=256, dtype=BF16),
    # backward (training) pass of the scan at the headline layer and at the training-step
    # sweep's shape (batch 8, d_model 256 -> 512 channels, 32K tokens)
    "scan_bwd_bf16_B1_L4096_D1536_N16": dict(kind="scan_bwd", B=1, L=4096, D=1536, N=16, dtype=BF16),
    "scan_bwd_bf16_B8_L32768_D512_N16": dict(kind="scan_bwd", B=8, L=32768, D=512, N=16, dtype=BF16),
    # ... and at N = 64 of the state-dimension sweep (chunks of 16 states)
    "scan_bwd_bf16_B1_L4096_D1536_N64": dict(kind="scan_bwd", B=1, L=4096, D=1536, N=64, dtype=BF16),
    # the headline layer with exact zero-order hold and softplus(delta + bias) in the kernel
    "scan_zoh_softplus_bf16_B1_L4096_D1536_N16": dict(kind="scan_var", B=1, L=4096, D=1536, N=16, dtype=BF16),
    "scan_zoh_softplus_bf16_B1_L4096_D1536_N64": dict(kind="scan_var", B=1, L=4096, D=1536, N=64, dtype=BF16),
    # the headline layer as a Mamba-3 scan (complex transitions, exponential-trapezoidal rule)
    "scan3_bf16_B1_L4096_D1536_N16": dict(kind="scan3", B=1, L=4096, D=1536, N=16, dtype=BF16),
    "ssd_bf16_B4_L8192_H24_P64_N128_Q256": dict(kind="ssd", B=4, L=8192, H=24, P=64, N=128,
                                                chunk=256, dtype=BF16),
    "ssd_bf16_B4_L8192_H24_P64_N128_Q64": dict(kind="ssd", B=4, L=8192, H=24, P=64, N=128,
                                               chunk=64, dtype=BF16),
    "ssd_bf16_B4_L8000_H24_P64_N128_Q256": dict(kind="ssd", B=4, L=8000, H=24, P=64, N=128,
                                                chunk=256, dtype=BF16),
    "step_bf16_B64_D3072_N16_x1000": dict(kind="step", B=64, D=3072, N=16, steps=1000, dtype=BF16),
    # Mamba-2 decode (a Mamba2-130m-sized layer: 24 heads of 64, N = 128), 200 steps in place
    "ssd_step_bf16_B64_H24_P64_N128_x200": dict(kind="ssd_step", B=64, H=24, P=64, N=128, steps=200,
                                                dtype=BF16),
    # Mamba-3 decode at the Mamba-1 decode layer's size (complex state: 25.2 MB), 200 steps in place
    "step3_bf16_B64_D3072_N16_x200": dict(kind="step3", B=64, D=3072, N=16, steps=200, dtype=BF16),
}
