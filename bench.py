"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--no-cpu] [--no-other]

A step is one ssm_scan_fwd call over one batch of synthetic input already
resident in HBM (bf16 I/O, B=1, L=4096, D=1536, N=16 by default). Inputs rotate
over several independent batches whose total size exceeds the 256 MB
last-level (MALL) cache, so every step streams its batch from HBM.

Prints ONE JSON line: throughput in state updates/s (B*L*D*N per step), the
roofline of the dominant kernel (timed live with HIP events recorded around
each kernel launch on the launch stream), and the fp64 oracle timed on the
host cores on a bounded sample of the same workload. ``other_paths`` holds the
same measurements for the long-sequence scan, the state-dimension sweep, the
backward (training) scan, the SSD and the two decode steps.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks and unit counts
HBM_PEAK_GBS = 8000.0
CUS, LANES, CLOCK_GHZ = 256, 64, 2.4
LANE_SLOTS_PER_S = CUS * LANES * CLOCK_GHZ * 1e9      # one fp32 VALU op per lane per clock
MFMA_BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
# per state update the minimal instruction mix: v_mul (Delta*A), v_exp_f32 (half
# rate: 2 lane-slots), v_mul (u*B), v_fma (state), v_fma (C.h) -> 6 lane-slots
SLOTS_PER_UPDATE = 6.0


def hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    return lib


class KernelTimer:
    """HIP events the library hands to the runtime with every kernel launch it
    makes: a (start, stop) pair per kernel, stamped at the kernel's own start and end."""

    def __init__(self, n):
        self.h = hip()
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            assert self.h.hipEventCreate(ctypes.byref(e)) == 0
            self.ev[i] = e
        self.n = n

    def start(self, lib):
        lib.ssm_profile_events.argtypes = [ctypes.c_void_p, ctypes.c_int]
        lib.ssm_profile_events(ctypes.cast(self.ev, ctypes.c_void_p), self.n)

    def stop(self, lib):
        return lib.ssm_profile_events(None, 0)

    def elapsed_ms(self, i, j):
        self.h.hipEventSynchronize(self.ev[j])
        ms = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[j]) == 0
        return ms.value

    def close(self):
        for i in range(self.n):
            self.h.hipEventDestroy(self.ev[i])


def sync():
    import torch
    torch.cuda.synchronize()


# ------------------------------------------------------------------ scan
def scan_setup(wl, dev, max_sets=16):
    import torch
    import ssm_inputs as si
    import selective_scan_amd as ssa
    B, L, D, N = wl["B"], wl["L"], wl["D"], wl["N"]
    es = 2 if wl["dtype"] == si.BF16 else 4
    set_bytes = 4 * B * L * D * es + 2 * B * L * N * es
    R = max(1, min(max_sets, math.ceil(2 * MALL_BYTES / set_bytes)))
    sets = []
    for r in range(R):
        w = si.scan_inputs(B, L, D, N, dtype=wl["dtype"], seed=r)
        t = {k: si.to_torch(w[k], dev) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D")}
        t["y"] = torch.empty_like(t["x"])
        t["hf"] = torch.empty((B, D, N), dtype=torch.float32, device=dev)
        sets.append(t)
        if r == 0:
            w0 = w
    ws_bytes = ssa.ssm_scan_workspace_size(B, L, D, N)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    return sets, ws, w0, set_bytes


def scan_call(t, ws):
    import selective_scan_amd as ssa
    ssa.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"],
                     y=t["y"], h_final=t["hf"], workspace=ws)


def scan_alg_bytes(wl):
    """Algorithmic HBM bytes per call: read x, Delta, z, B, C, A, D; write y, h_final."""
    B, L, D, N = wl["B"], wl["L"], wl["D"], wl["N"]
    es = 2 if wl["dtype"] == "bf16" else 4
    return 4 * B * L * D * es + 2 * B * L * N * es + (D * N + D) * 4 + B * D * N * 4


def count_kernels(call):
    """Kernels one call launches: the library uses two events per launch."""
    import selective_scan_amd as ssa
    lib = ssa.ops.lib()
    kt = KernelTimer(64)
    kt.start(lib)
    call()
    used = kt.stop(lib)
    sync()
    kt.close()
    return used // 2


def time_calls(call, sets, steps, warmup, n_kernels):
    """Time `steps` calls (rotating over `sets`) between two events on the launch
    stream; then time every kernel of another `steps` calls with the library's
    profiling events (kept out of the throughput run: an event record between two
    launches adds a dispatch gap)."""
    import torch
    import selective_scan_amd as ssa
    lib = ssa.ops.lib()
    for i in range(warmup):
        call(sets[i % len(sets)])
    sync()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        call(sets[(warmup + i) % len(sets)])
    t1.record()
    sync()
    total_ms = t0.elapsed_time(t1)
    kt = KernelTimer(steps * 2 * n_kernels)
    kt.start(lib)
    for i in range(steps):
        call(sets[(warmup + steps + i) % len(sets)])
    used = kt.stop(lib)
    sync()
    per_k = 2 * n_kernels
    assert used == steps * per_k, f"recorded {used} events, expected {steps * per_k}"
    ker = np.array([[kt.elapsed_ms(s * per_k + 2 * k, s * per_k + 2 * k + 1) for k in range(n_kernels)]
                    for s in range(steps)])
    kt.close()
    return total_ms, ker


# Sources each kernel is compiled from, in the order their bytes are hashed.
KERNEL_SOURCES = {
    "scan": ("scan_core.h", "scan_fwd.hip", "common.h", "launch.h"),
    "scan_var": ("scan_core.h", "scan_var.hip", "common.h", "launch.h"),
    "scan_bwd": ("scan_bwd.hip", "common.h", "launch.h"),
    "ssd": ("ssd_fwd.hip", "common.h", "launch.h"),
}


def _code_only(text):
    """C++ source without comments and with runs of whitespace collapsed: what the
    compiler sees (string literals in these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def sources_sha256(kind):
    """SHA-256 of a kernel's sources (KERNEL_SOURCES, in order), comments and
    whitespace excluded: a comment edit does not void a measurement."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "selective_scan_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def committed_traffic(kind, summary):
    """HBM bytes per launch (or per call), from a committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary under profiles/ -- only while the kernel's
    sources are byte-identical to the ones the counters were taken on."""
    import re
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    m_h = re.search(r"sources_sha256:\s*([0-9a-f]{64})", text)
    if not (m_b and m_h):
        return None
    return int(m_b.group(1)) if sources_sha256(kind) == m_h.group(1) else None


def scan_bench(name, wl, steps, warmup, dev):
    sets, ws, w0, set_bytes = scan_setup(wl, dev)
    nk = count_kernels(lambda: scan_call(sets[0], ws))
    total_ms, ker = time_calls(lambda t: scan_call(t, ws), sets, steps, warmup, nk)
    upd = wl["B"] * wl["L"] * wl["D"] * wl["N"]
    ms = total_ms / steps
    kmean = ker.mean(axis=0)
    dom = int(np.argmax(kmean))
    alg = scan_alg_bytes(wl)
    res = dict(
        workload=name, ms_per_step=ms, updates_per_s=upd / (ms * 1e-3),
        tokens_per_s=wl["B"] * wl["L"] / (ms * 1e-3),
        hbm_gbs=alg / (ms * 1e-3) / 1e9, hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        kernel_ms=[float(v) for v in kmean], dominant_kernel=dom, sets=len(sets),
        set_mb=set_bytes / 1e6,
    )
    tdom = kmean[dom] * 1e-3
    achieved = SLOTS_PER_UPDATE * upd / tdom / 1e12
    peak = LANE_SLOTS_PER_S / 1e12
    res["roofline"] = dict(bound="alu", achieved=achieved, peak=peak, unit="Tslot/s",
                           frac=achieved / peak, traffic=committed_traffic("scan", f"traffic_{name}.md"),
                           kernel="segment_final" if nk > 1 else "segment")
    res["hbm_roofline_dominant"] = dict(achieved=alg / tdom / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                                        frac=alg / tdom / 1e9 / HBM_PEAK_GBS)
    return res, w0


def scan_cpu_baseline(wl, w0, budget_s=15.0, total_s=10.0):
    """The fp64 oracle (as it stands) on the host cores: whole sequences of as many
    channels as fit in about `budget_s` seconds (all of them when they fit), run
    again until about `total_s` seconds of work have been timed; the median run."""
    import oracle
    import ssm_inputs as si
    o = oracle.get()
    o.set_threads(len(os.sched_getaffinity(0)))
    T = o.get_threads()
    f = {k: si.to_f64(w0[k]) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D")}
    B, L, D, N = wl["B"], wl["L"], wl["D"], wl["N"]

    def run(dsel):
        sl = slice(0, dsel)
        c = lambda a: np.ascontiguousarray(a[:, :, sl])
        t0 = time.perf_counter()
        o.scan(c(f["x"]), c(f["delta"]), np.ascontiguousarray(f["A"][sl]), f["Bm"], f["Cm"],
               D=np.ascontiguousarray(f["D"][sl]), z=c(f["z"]))
        return time.perf_counter() - t0

    probe = run(min(D, T))                       # one channel per thread
    dsel = int(min(D, max(T, budget_s / max(probe, 1e-6) * T * 0.7)))
    reps, els = 0, []
    while reps < 1000 and (reps < 3 or sum(els) < total_s):
        els.append(run(dsel))
        reps += 1
    el = float(np.median(els))
    upd = B * L * dsel * N
    return dict(value=upd / el, unit="state updates/s", cores=T, kind="oracle",
                sample=f"fp64 oracle (sequential recurrence) on B={B}, L={L}, {dsel} of {D} channels, "
                       f"N={N}: {upd / 1e6:.1f} M updates, median of {reps} run(s), {el:.3f} s each")


# ------------------------------------------------------------------ scan variants
# Exact zero-order hold per state update (steps whose |z| are all >= 1/32): v_mul
# (Delta*A), v_exp_f32 (2), v_mul (x/A), v_mul (*B), v_add (h + w), v_fma (state),
# v_fma (C.h) -> 8 lane-slots; softplus(delta + bias) is per (step, channel), not
# per update.
ZOH_SLOTS_PER_UPDATE = 8.0


def scan_var_bench(name, wl, steps, warmup, dev, max_sets=16):
    import torch
    import ssm_inputs as si
    import selective_scan_amd as ssa
    B, L, D, N = wl["B"], wl["L"], wl["D"], wl["N"]
    es = 2 if wl["dtype"] == si.BF16 else 4
    set_bytes = 4 * B * L * D * es + 2 * B * L * N * es
    R = max(1, min(max_sets, math.ceil(2 * MALL_BYTES / set_bytes)))
    sets = []
    for r in range(R):
        w = si.scan_inputs(B, L, D, N, dtype=wl["dtype"], seed=r)
        raw = si.scan_raw_delta(B, L, D, dtype=wl["dtype"], seed=r)
        t = {k: si.to_torch(w[k], dev) for k in ("x", "z", "Bm", "Cm", "A", "D")}
        t["delta"] = si.to_torch(raw["delta"], dev)
        t["bias"] = torch.from_numpy(raw["delta_bias"]).to(dev)
        t["y"] = torch.empty_like(t["x"])
        t["hf"] = torch.empty((B, D, N), dtype=torch.float32, device=dev)
        sets.append(t)
    ws = torch.empty(max(ssa.ssm_scan_workspace_size(B, L, D, N), 1), dtype=torch.uint8, device=dev)

    def call(t):
        ssa.ssm_scan_fwd_ex(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], D=t["D"], z=t["z"], disc="zoh",
                            delta_bias=t["bias"], delta_softplus=True, y=t["y"], h_final=t["hf"], workspace=ws)

    nk = count_kernels(lambda: call(sets[0]))
    total_ms, ker = time_calls(call, sets, steps, warmup, nk)
    ms = total_ms / steps
    kmean = ker.mean(axis=0)
    dom = int(np.argmax(kmean))
    upd = B * L * D * N
    alg = scan_alg_bytes(wl) + D * 4
    achieved = ZOH_SLOTS_PER_UPDATE * upd / (kmean[dom] * 1e-3) / 1e12
    peak = LANE_SLOTS_PER_S / 1e12
    return dict(workload=name, ms_per_step=ms, updates_per_s=upd / (ms * 1e-3), tokens_per_s=B * L / (ms * 1e-3),
                kernel_ms=[float(v) for v in kmean], hbm_gbs=alg / (ms * 1e-3) / 1e9,
                hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, sets=len(sets),
                roofline=dict(bound="alu", achieved=achieved, peak=peak, unit="Tslot/s", frac=achieved / peak,
                              traffic=committed_traffic("scan_var", f"traffic_{name}.md"),
                              kernel="segment_final (zero-order hold, softplus(delta + bias))"))


# ------------------------------------------------------------------ scan backward
# Per state update, the final backward pass must issue (non-packed VALU lane-slots):
# forward recompute v_mul (Delta*A), v_exp_f32 (2), v_mul (u*B), v_fma (state),
# v_fma (C.h), v_mul (dv*h for dC); backward v_fma (adjoint), v_mul + v_exp_f32 (2)
# (decay again), v_fma (a_t h_{t-1}), v_mul (q), v_fma x 3 (ddelta, dA, dx sums),
# v_mul (g*u for dB), v_mul (carry) -> 18; plus the sums over the 64 channels of a
# wave for dB and dC, at least 2 x 63/64 adds -> 20 lane-slots per update.
BWD_SLOTS_PER_UPDATE = 20.0


def scan_bwd_bench(name, wl, steps, warmup, dev, max_sets=8):
    import torch
    import ssm_inputs as si
    import selective_scan_amd as ssa
    B, L, D, N = wl["B"], wl["L"], wl["D"], wl["N"]
    es = 2 if wl["dtype"] == si.BF16 else 4
    set_bytes = 4 * B * L * D * es + 2 * B * L * N * es
    R = max(1, min(max_sets, math.ceil(2 * MALL_BYTES / set_bytes)))
    sets = []
    for r in range(R):
        w = si.scan_inputs(B, L, D, N, dtype=wl["dtype"], seed=r)
        gw = si.scan_grad_inputs(B, L, D, N, dtype=wl["dtype"], seed=r)
        t = {k: si.to_torch(w[k], dev) for k in ("x", "delta", "z", "Bm", "Cm", "A", "D")}
        t["dy"] = si.to_torch(gw["dy"], dev)
        t["dhf"] = si.to_torch(gw["dh_final"], dev)
        t["out"] = dict(dx=torch.empty_like(t["x"]), ddelta=torch.empty_like(t["x"]), dz=torch.empty_like(t["x"]),
                        dA=torch.empty_like(t["A"]), dBm=torch.empty_like(t["Bm"]), dCm=torch.empty_like(t["Cm"]),
                        dD=torch.empty_like(t["D"]), dh0=torch.empty((B, D, N), dtype=torch.float32, device=dev))
        sets.append(t)
    ws = torch.empty(max(ssa.ssm_scan_bwd_workspace_size(B, L, D, N), 1), dtype=torch.uint8, device=dev)

    def call(t):
        ssa.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], D=t["D"], z=t["z"],
                         dh_final=t["dhf"], out=t["out"], workspace=ws)

    nk = count_kernels(lambda: call(sets[0]))
    total_ms, ker = time_calls(call, sets, steps, warmup, nk)
    ms = total_ms / steps
    kmean = ker.mean(axis=0)
    dom = int(np.argmax(kmean))
    upd = B * L * D * N
    # algorithmic bytes: read x, Delta, z, dy, B, C, A, D, dh_final; write dx, ddelta, dz,
    # dB, dC, dA, dD, dh0
    alg = 7 * B * L * D * es + 4 * B * L * N * es + 2 * (D * N + D) * 4 + 2 * B * D * N * 4
    tdom = kmean[dom] * 1e-3
    achieved = BWD_SLOTS_PER_UPDATE * upd / tdom / 1e12
    peak = LANE_SLOTS_PER_S / 1e12
    return dict(workload=name, ms_per_step=ms, updates_per_s=upd / (ms * 1e-3),
                tokens_per_s=B * L / (ms * 1e-3), kernel_ms=[float(v) for v in kmean],
                hbm_gbs=alg / (ms * 1e-3) / 1e9, hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                sets=len(sets), alg_bytes=alg,
                roofline=dict(bound="alu", achieved=achieved, peak=peak, unit="Tslot/s", frac=achieved / peak,
                              traffic=committed_traffic("scan_bwd", f"traffic_{name}.md"),
                              kernel="bwd_final"))


# ------------------------------------------------------------------ SSD
def ssd_alg(wl):
    """Algorithmic HBM bytes and dense matrix flops per call.
    bytes: read x, Delta, B, C, A; write y, h_final.
    flops: G = C B^T once per (batch, chunk) (shared by the heads), and per
    (batch, head, chunk) M X, the chunk state and C H: 2QQN + H(2QQP + 4QNP)."""
    B, L, H, P, N, Q = wl["B"], wl["L"], wl["H"], wl["P"], wl["N"], wl["chunk"]
    byt = 2 * (2 * B * L * H * P) + 2 * B * L * H + 2 * 2 * B * L * N + 4 * H + 4 * B * H * N * P
    fl = 0.0
    for c0 in range(0, L, Q):
        q = min(Q, L - c0)
        fl += B * (2.0 * q * q * N + H * (2.0 * q * q * P + 4.0 * q * N * P))
    return byt, fl


def ssd_bench(name, wl, steps, warmup, dev, max_sets=3):
    import torch
    import selective_scan_amd as ssa
    import ssm_inputs as si
    B, L, H, P, N, Q = wl["B"], wl["L"], wl["H"], wl["P"], wl["N"], wl["chunk"]
    sets = []
    for r in range(max_sets):
        w = si.ssd_inputs(B, L, H, P, N, seed=r)
        t = {k: si.to_torch(w[k], dev) for k in ("x", "delta", "Bm", "Cm", "A")}
        t["y"] = torch.empty_like(t["x"])
        t["hf"] = torch.empty((B, H, N, P), dtype=torch.float32, device=dev)
        sets.append(t)
    need = ssa.ssm_ssd_workspace_size(B, L, H, P, N, Q)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def call(t):
        ssa.ssm_ssd_fwd(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], chunk=Q, y=t["y"],
                        h_final=t["hf"], workspace=ws)

    nk = count_kernels(lambda: call(sets[0]))
    total_ms, ker = time_calls(call, sets, steps, warmup, nk)
    ms = total_ms / steps
    kmean = ker.mean(axis=0)
    byt, fl = ssd_alg(wl)
    upd = B * L * H * P * N
    tdom = kmean[int(np.argmax(kmean))] * 1e-3
    return dict(workload=name, ms_per_step=ms, updates_per_s=upd / (ms * 1e-3),
                tokens_per_s=B * L / (ms * 1e-3), kernel_ms=[float(v) for v in kmean],
                hbm_gbs=byt / (ms * 1e-3) / 1e9, hbm_frac=byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                mfma_tflops=fl / (ms * 1e-3) / 1e12,
                mfma_frac=fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                roofline=dict(bound="hbm", achieved=byt / (ms * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              traffic=committed_traffic("ssd", f"ssd_kernels_{name[4:]}.md"),
                              kernel="whole call (three kernels)"),
                dominant_kernel_ms=tdom * 1e3, alg_bytes=byt, alg_flops=fl)


# ------------------------------------------------------------------ decode
def step_bench(wl, dev, reps=3):
    import torch
    import selective_scan_amd as ssa
    import ssm_inputs as si
    B, D, N, steps = wl["B"], wl["D"], wl["N"], wl["steps"]
    w = si.step_inputs(B, D, N, steps=steps, dtype=wl["dtype"], seed=0)
    tok = {k: si.to_torch(w[k], dev) for k in ("x", "delta", "z", "Bm", "Cm")}
    A = torch.from_numpy(w["A"]).to(dev)
    Dk = torch.from_numpy(w["D"]).to(dev)
    st0 = torch.from_numpy(w["state0"]).to(dev)
    st = st0.clone()
    y = torch.empty((steps, B, D), dtype=tok["x"].dtype, device=dev)

    def run():
        for s in range(steps):
            ssa.ssm_step(st, tok["x"][s], tok["delta"][s], A, tok["Bm"][s], tok["Cm"][s], D=Dk,
                         z=tok["z"][s], y=y[s])

    run()
    sync()
    times = []
    for _ in range(reps):
        st.copy_(st0)
        sync()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        sync()
        times.append(e0.elapsed_time(e1))
    # HIP-graph replay of the same 1000 launches
    g = torch.cuda.CUDAGraph()
    st.copy_(st0)
    sync()
    s_ = torch.cuda.Stream()
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            run()
    sync()
    gtimes = []
    for _ in range(reps):
        st.copy_(st0)
        sync()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        sync()
        gtimes.append(e0.elapsed_time(e1))
    es = 2 if wl["dtype"] == "bf16" else 4
    alg = 2 * B * D * N * 4 + 4 * B * D * es + 2 * B * N * es + (D * N + D) * 4
    med = float(np.median(times)) / steps
    gmed = float(np.median(gtimes)) / steps
    cold = cold_decode(lambda stv, s_: ssa.ssm_step(stv, tok["x"][s_], tok["delta"][s_], A, tok["Bm"][s_],
                                                    tok["Cm"][s_], D=Dk, z=tok["z"][s_], y=y[s_]),
                       st0, steps)
    return dict(workload="step_bf16_B64_D3072_N16_x1000", ms_per_step_stream=med,
                ms_per_step_graph=gmed, updates_per_s_graph=B * D * N / (gmed * 1e-3),
                tokens_per_s_graph=B / (gmed * 1e-3),
                hbm_gbs_graph=alg / (gmed * 1e-3) / 1e9,
                note="state (12.6 MB) stays resident in the 256 MB MALL across in-place steps",
                cold=dict(layers=cold["layers"], ms_per_step_graph=cold["ms"],
                          hbm_gbs_graph=alg / (cold["ms"] * 1e-3) / 1e9,
                          hbm_frac=alg / (cold["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          note="step s updates the state of layer s mod layers: the states "
                               "(%d x %.1f MB) exceed the MALL, so each step streams its state from HBM"
                               % (cold["layers"], st0.numel() * 4 / 1e6)),
                streaming_floor=streaming_floor(st0, steps))


def streaming_floor(st0, steps, reps=3):
    """Context for a decode step: a plain in-place scale of a tensor of the state's
    size (torch's mul_, one launch per step), graph-replayed `steps` times on one
    tensor (MALL-resident) and rotating over tensors adding up to more than the MALL.
    What one launch per step reaches by pure streaming at this size."""
    import torch
    st = st0.clone()
    g = torch.cuda.CUDAGraph()
    sync()
    s_ = torch.cuda.Stream()
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            for _ in range(steps):
                st.mul_(0.999)
    sync()
    hot = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        sync()
        hot.append(e0.elapsed_time(e1) / steps)
    cold = cold_decode(lambda stv, s_: stv.mul_(0.999), st0, steps, reps=reps)
    return dict(ms_per_step_hot=float(np.median(hot)), ms_per_step_cold=cold["ms"],
                bytes_per_step=2 * st0.numel() * 4,
                note="plain in-place scale of a tensor of the state's size (torch mul_), graph-replayed "
                     "like the steps: reads and writes the state only")


def cold_decode(step, st0, steps, reps=3, min_bytes=2 * MALL_BYTES):
    """A multi-layer decode: `steps` in-place steps, step s on the state of layer
    s mod R, with R states of st0's size adding up to more than the MALL; replayed
    from a HIP graph. Returns the median time per step."""
    import torch
    R = max(2, math.ceil(min_bytes / (st0.numel() * 4)))
    states = [st0.clone() for _ in range(R)]
    g = torch.cuda.CUDAGraph()
    sync()
    s_ = torch.cuda.Stream()
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            for s in range(steps):
                step(states[s % R], s)
    sync()
    out = []
    for _ in range(reps):
        for t in states:
            t.copy_(st0)
        sync()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        sync()
        out.append(e0.elapsed_time(e1) / steps)
    return dict(layers=R, ms=float(np.median(out)))


def ssd_step_bench(wl, dev, reps=3):
    """Mamba-2 decode: `steps` in-place steps launched on a stream, then the same
    steps replayed from a HIP graph; per-step time and algorithmic bytes/s."""
    import torch
    import selective_scan_amd as ssa
    import ssm_inputs as si
    B, H, P, N, steps = wl["B"], wl["H"], wl["P"], wl["N"], wl["steps"]
    w = si.ssd_step_inputs(B, H, P, N, steps=steps, dtype=wl["dtype"], seed=0)
    tok = {k: si.to_torch(w[k], dev) for k in ("x", "delta", "z", "Bm", "Cm")}
    A = torch.from_numpy(w["A"]).to(dev)
    Dk = torch.from_numpy(w["D"]).to(dev)
    st0 = torch.from_numpy(w["state0"]).to(dev)
    st = st0.clone()
    y = torch.empty((steps, B, H, P), dtype=tok["x"].dtype, device=dev)

    def run():
        for s in range(steps):
            ssa.ssm_ssd_step(st, tok["x"][s], tok["delta"][s], A, tok["Bm"][s], tok["Cm"][s], D=Dk,
                             z=tok["z"][s], y=y[s])

    def timed(fn):
        out = []
        for _ in range(reps):
            st.copy_(st0)
            sync()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            sync()
            out.append(e0.elapsed_time(e1) / steps)
        return float(np.median(out))

    run()
    sync()
    ms_stream = timed(run)
    g = torch.cuda.CUDAGraph()
    st.copy_(st0)
    sync()
    s_ = torch.cuda.Stream()
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            run()
    sync()
    ms_graph = timed(g.replay)
    es = 2 if wl["dtype"] == "bf16" else 4
    alg = 2 * B * H * N * P * 4 + 3 * B * H * P * es + B * H * es + 2 * B * N * es + 2 * H * 4
    cold = cold_decode(lambda stv, s_: ssa.ssm_ssd_step(stv, tok["x"][s_], tok["delta"][s_], A, tok["Bm"][s_],
                                                        tok["Cm"][s_], D=Dk, z=tok["z"][s_], y=y[s_]),
                       st0, steps)
    return dict(workload="ssd_step_bf16_B64_H24_P64_N128_x200", ms_per_step_stream=ms_stream,
                ms_per_step_graph=ms_graph, updates_per_s_graph=B * H * P * N / (ms_graph * 1e-3),
                tokens_per_s_graph=B / (ms_graph * 1e-3), alg_bytes_per_step=alg,
                hbm_gbs_graph=alg / (ms_graph * 1e-3) / 1e9,
                note="state (50.3 MB) stays resident in the 256 MB MALL across in-place steps",
                cold=dict(layers=cold["layers"], ms_per_step_graph=cold["ms"],
                          hbm_gbs_graph=alg / (cold["ms"] * 1e-3) / 1e9,
                          hbm_frac=alg / (cold["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          note="step s updates the state of layer s mod layers: the states "
                               "(%d x %.1f MB) exceed the MALL, so each step streams its state from HBM"
                               % (cold["layers"], st0.numel() * 4 / 1e6)),
                streaming_floor=streaming_floor(st0, steps))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="scan_bf16_B1_L4096_D1536_N16")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-other", action="store_true")
    ap.add_argument("--other", default=None,
                    help="only run this one other-paths workload (a scan_bwd_*, scan_zoh_* or ssd_* name) and print it")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the selective scan here has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import ssm_inputs as si
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        sync()
        print(json.dumps({"calibrate_copy_bytes_read": src.numel() * 4, "calibrate_copy_bytes_written": dst.numel() * 4,
                          "launches": 5}))
        return
    if args.other:
        wl = si.WORKLOADS[args.other]
        if wl["kind"] == "scan_bwd":
            r = scan_bwd_bench(args.other, wl, args.steps, args.warmup, dev)
        elif wl["kind"] == "scan_var":
            r = scan_var_bench(args.other, wl, args.steps, args.warmup, dev)
        elif wl["kind"] == "ssd":
            r = ssd_bench(args.other, wl, args.steps, args.warmup, dev)
        else:
            raise SystemExit(f"--other takes a scan_bwd_* or ssd_* workload, not {args.other}")
        print(json.dumps(r))
        return
    wl = si.WORKLOADS[args.workload]
    assert wl["kind"] == "scan", "the headline bench line is a scan workload"
    res, w0 = scan_bench(args.workload, wl, args.steps, args.warmup, dev)
    out = {
        "metric": "selective-scan state updates/s (B*L*D*N) + % of MI355X HBM roofline",
        "value": res["updates_per_s"],
        "unit": "state updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl["dtype"] == "f32" else "f32 (bf16 I/O)",
        "data": "synthetic (seeded; distributions of the pages' workloads)",
        "config": {"workload": args.workload, "B": wl["B"], "L": wl["L"], "D": wl["D"],
                   "N": wl["N"], "io": wl["dtype"], "rotating_input_sets": res["sets"]},
        "tokens_per_s": res["tokens_per_s"],
        "hbm_gbs": res["hbm_gbs"],
        "hbm_frac": res["hbm_frac"],
        "kernel_ms": res["kernel_ms"],
        "roofline": res["roofline"],
        "hbm_roofline_dominant": res["hbm_roofline_dominant"],
    }
    if not args.no_cpu:
        out["cpu_baseline"] = scan_cpu_baseline(wl, w0)
    if not args.no_other:
        other = {}
        r2, _ = scan_bench("scan_bf16_B8_L32768_D512_N16", si.WORKLOADS["scan_bf16_B8_L32768_D512_N16"],
                           steps=5, warmup=2, dev=dev)
        other["scan_long"] = {k: r2[k] for k in ("workload", "ms_per_step", "updates_per_s", "tokens_per_s",
                                                   "hbm_gbs", "hbm_frac", "kernel_ms", "roofline")}
        for nm in ("scan_bf16_B1_L4096_D1536_N64", "scan_bf16_B1_L4096_D1536_N128",
                   "scan_bf16_B1_L4096_D1536_N256"):
            r3, _ = scan_bench(nm, si.WORKLOADS[nm], steps=10, warmup=2, dev=dev)
            other[nm] = {k: r3[k] for k in ("workload", "ms_per_step", "updates_per_s", "tokens_per_s",
                                            "hbm_gbs", "hbm_frac", "kernel_ms", "roofline")}
        other["scan_zoh_softplus_bf16_B1_L4096_D1536_N16"] = scan_var_bench(
            "scan_zoh_softplus_bf16_B1_L4096_D1536_N16", si.WORKLOADS["scan_zoh_softplus_bf16_B1_L4096_D1536_N16"],
            steps=20, warmup=3, dev=dev)
        for nm in ("scan_bwd_bf16_B1_L4096_D1536_N16", "scan_bwd_bf16_B8_L32768_D512_N16"):
            other[nm] = scan_bwd_bench(nm, si.WORKLOADS[nm], steps=10 if si.WORKLOADS[nm]["L"] <= 4096 else 3,
                                       warmup=2, dev=dev)
        for nm in ("ssd_bf16_B4_L8192_H24_P64_N128_Q256", "ssd_bf16_B4_L8192_H24_P64_N128_Q64",
                   "ssd_bf16_B4_L8000_H24_P64_N128_Q256"):
            other[nm] = ssd_bench(nm, si.WORKLOADS[nm], steps=10, warmup=3, dev=dev)
        other["decode"] = step_bench(si.WORKLOADS["step_bf16_B64_D3072_N16_x1000"], dev)
        other["ssd_decode"] = ssd_step_bench(si.WORKLOADS["ssd_step_bf16_B64_H24_P64_N128_x200"], dev)
        out["other_paths"] = other
    print(json.dumps(out))


if __name__ == "__main__":
    main()
