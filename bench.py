"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--no-cpu] [--no-other]
    python bench.py --valu-rates | --calibrate-copy | --other NAME

A step is one ssm_scan_fwd call over one batch of synthetic input already
resident in HBM. The default workload is the long-sequence scan (bf16 I/O,
B=8, L=32768, D=512, N=16: 1.09 GB per call, more than four times the 256 MB
last-level (MALL) cache, so every step streams from HBM).

Prints ONE JSON line: throughput in state updates/s (B*L*D*N per step) over K
back-to-back steps, the median and P95 of at least 100 individually timed calls,
the HBM roofline of the dominant kernel and of the whole call (algorithmic bytes
over time; every kernel timed live with HIP events the runtime stamps at the
kernel's own start and end), the VALU issue figures from committed rocprofv3
instruction counters, the fp64 oracle timed on the host cores on a bounded
sample of the same workload, and the pages' own published figures as context.
``other_paths`` holds the small fp32 case, the Mamba-130m-sized layer, the
state-dimension sweep, the zero-order-hold variant, the backward scan, the SSD,
the two decode steps, and the VALU issue-rate probes.
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
# fp32 vector peak 157.3 TFLOP/s = 256 CU x 128 FMA lanes per clock x 2 flops x 2.4 GHz: a
# wave64 v_fma_f32 (non-packed) issues in two cycles per SIMD, as the VALU-rate probe
# confirms. One lane-slot = one fp32 FMA-class op of one lane.
FMA_LANES_PER_CU_CLK = 128
LANE_SLOTS_PER_S = CUS * FMA_LANES_PER_CU_CLK * CLOCK_GHZ * 1e9   # 78.6e12
MFMA_BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
# Non-transcendental VALU ops per state update that one pass of the recurrence needs:
# v_mul (Delta*A), v_mul (u*B), v_fma (state), v_fma (C.h); plus one v_exp_f32, priced at the
# transcendental issue cost the VALU-rate probes measure (about 3.8 slots on the MI355X).
FMA_OPS_PER_UPDATE = 4.0
DEFAULT_TRANS_COST = 3.8
DEFAULT_WORKLOAD = "scan_bf16_B8_L32768_D512_N16"
LATENCY_CALLS = 100

# The pages' own figures (other hardware, other implementations): context, never the target.
PAGE_CONTEXT = {
    "note": "published by the pages for naive per-timestep implementations on NVIDIA parts; "
            "context only, not comparable kernels and not the target",
    "ssm_bench_bandwidth_utilisation": {
        "value": "0.01-0.08 % of peak (A100-SXM4-40GB), 0.02-0.15 % of peak (Tesla T4)",
        "what": "Python-loop selective-scan SSM, one kernel launch per time step, bf16, batch 1, "
                "L 512-4096, state dims 64/128/256",
        "source": "ssm-bench README, status table"},
    "s4d_train_step_32k": {
        "value": "13.5 s per training step at 32K tokens", "hardware": "RTX 4050 Laptop (6 GB)",
        "what": "S4D (FFT convolution; not the selective scan), batch 8, d_model 256, 2 layers",
        "source": "Efficient Sequence Modeling: From S4 to Mamba-3, section 06 Results"},
    "mamba1_python_loop_train_step": {
        "value": "2632 ms per training step at 1K tokens; 248 s at 4K", "hardware": "RTX 4050 Laptop (6 GB)",
        "what": "Python-loop Mamba-1 selective scan, batch 8, d_model 256, 2 layers",
        "source": "Efficient Sequence Modeling: From S4 to Mamba-3, section 06 Results"},
}


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


def warm_ms(call, s, steps=20, warmup=3):
    """Milliseconds per call with one input set called over and over: the set stays
    in the 256 MB MALL when it fits (the warm figure beside the cold, rotating one)."""
    import torch
    for _ in range(warmup):
        call(s)
    sync()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        call(s)
    t1.record()
    sync()
    return t0.elapsed_time(t1) / steps


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


def latency(call, sets, n=LATENCY_CALLS):
    """`n` calls, each between its own pair of events on the launch stream (rotating
    over `sets`): median and P95 of the per-call time, in ms."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    sync()
    for i, (a, b) in enumerate(ev):
        a.record()
        call(sets[i % len(sets)])
        b.record()
    sync()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return dict(median_ms=float(np.median(t)), p95_ms=float(np.percentile(t, 95)), min_ms=float(t.min()),
                calls=n)


# Sources each kernel is compiled from, in the order their bytes are hashed.
KERNEL_SOURCES = {
    "scan": ("scan_core.h", "scan_fwd.hip", "common.h", "launch.h"),
    "scan_var": ("scan_core.h", "scan_var.hip", "common.h", "launch.h"),
    "scan_bwd": ("scan_bwd.hip", "common.h", "launch.h"),
    "scan3": ("scan3.hip", "scan3.h", "common.h", "launch.h"),
    "step3": ("step3.hip", "step3.h", "common.h", "launch.h"),
    "ssd": ("ssd_fwd.hip", "common.h", "launch.h"),
    "step": ("step.hip", "common.h", "launch.h"),
    "ssd_step": ("ssd_step.hip", "common.h", "launch.h"),
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


def committed_valu(kind, summary):
    """Per-kernel VALU and transcendental instruction counts per launch (wave
    instructions, from rocprofv3 SQ_INSTS_VALU and SQ_INSTS_VALU_TRANS_F32) from a
    committed summary under profiles/, only while the kernel's sources are unchanged.
    Returns {kernel: (valu, trans)} or None."""
    import re
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"sources_sha256:\s*([0-9a-f]{64})", text)
    if not m_h or sources_sha256(kind) != m_h.group(1):
        return None
    out = {}
    for m in re.finditer(r"valu_insts_per_launch\s+(\S+):\s*(\d+)\s+trans_insts_per_launch:\s*(\d+)", text):
        out[m.group(1)] = (int(m.group(2)), int(m.group(3)))
    return out or None


def one_pass_slots(trans_cost):
    return FMA_OPS_PER_UPDATE + trans_cost


def alu_figures(counts, names, kmean_ms, t_call_ms, updates, trans_cost, one_pass=None, one_pass_note=None):
    """VALU issue per kernel and for the call from committed instruction counts: a
    wave instruction is 64 lane-slots, a transcendental one `trans_cost` times that
    (its issue rate relative to an FMA, measured by the VALU-rate probes). one_pass:
    the minimal single-pass mix in lane-slots per update (default: the Mamba-1 one)."""
    if counts is None:
        return None
    one = one_pass if one_pass is not None else one_pass_slots(trans_cost)
    per, tot = {}, 0.0
    for nm, t in zip(names, kmean_ms):
        if nm not in counts:
            continue
        valu, trans = counts[nm]
        slots = LANES * (valu + (trans_cost - 1.0) * trans)
        tot += slots
        per[nm] = dict(valu_insts=valu, trans_insts=trans, slots_per_update=slots / updates,
                       issue_tslot_s=slots / (t * 1e-3) / 1e12,
                       issue_frac=slots / (t * 1e-3) / LANE_SLOTS_PER_S)
    return dict(peak_tslot_s=LANE_SLOTS_PER_S / 1e12, trans_cost_slots=trans_cost, kernels=per,
                call_slots_per_update=tot / updates,
                call_issue_frac=tot / (t_call_ms * 1e-3) / LANE_SLOTS_PER_S,
                model_slots_per_update_one_pass=one,
                call_frac_of_one_pass_ceiling=one * updates / (t_call_ms * 1e-3) / LANE_SLOTS_PER_S,
                note="lane-slots = 64 x (VALU instructions + (trans_cost - 1) x transcendental ones), from "
                     "rocprofv3 SQ_INSTS_VALU / SQ_INSTS_VALU_TRANS_F32 per launch; issue_frac = slots over "
                     "kernel time x 256 CU x 128 FMA lanes x 2.4 GHz; call_frac_of_one_pass_ceiling = the "
                     "minimal single-pass mix (%s) over the call's time"
                     % (one_pass_note or "4 FMA-class ops + one exp per update"))


def scan_kernel_names(nk, wl):
    if nk == 3:  # N = 64, 128: the chunked final pass finishes y itself
        return ["segment_aggregate", "group_carry", "segment_final_sink" if wl["N"] >= 64 else "segment_final"]
    if nk == 2:
        return ["segment_aggregate", "segment_final"]
    if nk == 4:  # N = 256: two groups of state chunks, their sums added by a combine pass
        return ["segment_aggregate", "group_carry", "segment_final_sink", "combine_partials"]
    return ["segment_final"] if nk == 1 else [f"kernel{i}" for i in range(nk)]


def scan_bench(name, wl, steps, warmup, dev, trans_cost=DEFAULT_TRANS_COST, lat_calls=LATENCY_CALLS):
    sets, ws, w0, set_bytes = scan_setup(wl, dev)
    nk = count_kernels(lambda: scan_call(sets[0], ws))
    total_ms, ker = time_calls(lambda t: scan_call(t, ws), sets, steps, warmup, nk)
    lat = latency(lambda t: scan_call(t, ws), sets, max(lat_calls, steps))
    upd = wl["B"] * wl["L"] * wl["D"] * wl["N"]
    ms = total_ms / steps
    kmean = ker.mean(axis=0)
    names = scan_kernel_names(nk, wl)
    dom = int(np.argmax(kmean))
    alg = scan_alg_bytes(wl)
    res = dict(
        workload=name, ms_per_step=ms, updates_per_s=upd / (ms * 1e-3),
        tokens_per_s=wl["B"] * wl["L"] / (ms * 1e-3),
        hbm_gbs=alg / (ms * 1e-3) / 1e9, hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        call_latency=lat, kernel_ms=dict(zip(names, (float(v) for v in kmean))), dominant_kernel=names[dom],
        sets=len(sets), set_mb=set_bytes / 1e6, alg_bytes=alg,
        warm_ms_per_step=warm_ms(lambda t: scan_call(t, ws), sets[0]),
    )
    tdom = kmean[dom] * 1e-3
    traffic = committed_traffic("scan", f"traffic_{name}.md")
    res["roofline"] = dict(bound="hbm", achieved=alg / tdom / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                           frac=alg / tdom / 1e9 / HBM_PEAK_GBS, traffic=traffic, kernel=names[dom],
                           call=dict(achieved=alg / (ms * 1e-3) / 1e9, frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS),
                           note="achieved = the call's algorithmic bytes (x, Delta, z, B, C, A, D read; y, "
                                "h_final written) over the dominant kernel's mean time; 'call' over the whole "
                                "call. The scan at N = 16 is bound by VALU issue, not HBM: see 'alu'")
    res["alu"] = alu_figures(committed_valu("scan", f"valu_{name}.md"), names, kmean, ms, upd, trans_cost)
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
    # one thread on a slice sized to about 2 s
    o.set_threads(1)
    d1 = int(max(1, min(D, 2.0 / max(probe * T / min(D, T), 1e-6))))
    e1 = run(d1)
    o.set_threads(T)
    return dict(value=upd / el, unit="state updates/s", cores=T, kind="oracle",
                sample=f"fp64 oracle (sequential recurrence) on B={B}, L={L}, {dsel} of {D} channels, "
                       f"N={N}: {upd / 1e6:.1f} M updates, median of {reps} run(s), {el:.3f} s each",
                cpu_model=cpu_model(),
                single_thread=dict(value=B * L * d1 * N / e1, unit="state updates/s",
                                   sample=f"{d1} of {D} channels, one run of {e1:.2f} s"))


def device_info(dev):
    import torch
    p = torch.cuda.get_device_properties(dev)
    return dict(name=p.name, arch=getattr(p, "gcnArchName", None), compute_units=p.multi_processor_count,
                memory_gb=round(p.total_memory / 1e9, 1))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------ scan variants
# Exact zero-order hold per state update (steps whose |z| are all >= 1/32): v_mul
# (Delta*A), v_mul (x/A), v_mul (*B), v_add (h + w), v_fma (state), v_fma (C.h) -> 6
# FMA-class ops and one v_exp_f32; softplus(delta + bias) is per (step, channel), not
# per update.
ZOH_FMA_OPS_PER_UPDATE = 6.0


def scan_var_bench(name, wl, steps, warmup, dev, max_sets=16, trans_cost=DEFAULT_TRANS_COST):
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
    lat = latency(call, sets)
    ms = total_ms / steps
    kmean = ker.mean(axis=0)
    dom = int(np.argmax(kmean))
    upd = B * L * D * N
    alg = scan_alg_bytes(wl) + D * 4
    achieved = (ZOH_FMA_OPS_PER_UPDATE + trans_cost) * upd / (kmean[dom] * 1e-3) / 1e12
    peak = LANE_SLOTS_PER_S / 1e12
    return dict(workload=name, ms_per_step=ms, updates_per_s=upd / (ms * 1e-3), tokens_per_s=B * L / (ms * 1e-3),
                call_latency=lat, kernel_ms=[float(v) for v in kmean], hbm_gbs=alg / (ms * 1e-3) / 1e9,
                hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, sets=len(sets),
                roofline=dict(bound="alu", achieved=achieved, peak=peak, unit="Tslot/s", frac=achieved / peak,
                              traffic=committed_traffic("scan_var", f"traffic_{name}.md"),
                              kernel=("segment_final_sink" if N >= 64 else "segment_final")
                              + " (zero-order hold, softplus(delta + bias))"),
                alu=alu_figures(committed_valu("scan_var", f"valu_{name}.md"), scan_kernel_names(nk, wl), kmean,
                                ms, upd, trans_cost, one_pass=ZOH_FMA_OPS_PER_UPDATE + trans_cost,
                                one_pass_note="the fast zero-order-hold form: 6 FMA-class ops and one exp per update"))


# ------------------------------------------------------------------ Mamba-3 scan
# One pass of the Mamba-3 recurrence per state update: v_mul (Delta*Are), v_mul
# (Delta*theta), v_mul x 2 (|alpha| cos, |alpha| sin), v_fma (h + q B_{t-1}), v_mul (r B_t),
# v_fma x 2 (real part), v_mul + v_fma (imaginary part), v_fma (C.Re h) -> 11 FMA-class
# ops, and three transcendentals (v_exp_f32, v_sin_f32, v_cos_f32).
SCAN3_FMA_OPS_PER_UPDATE = 11.0
SCAN3_TRANS_PER_UPDATE = 3.0


def scan3_bench(name, wl, steps, warmup, dev, max_sets=16, trans_cost=DEFAULT_TRANS_COST):
    import torch
    import ssm_inputs as si
    import selective_scan_amd as ssa
    B, L, D, N = wl["B"], wl["L"], wl["D"], wl["N"]
    es = 2 if wl["dtype"] == si.BF16 else 4
    set_bytes = 5 * B * L * D * es + 2 * B * L * N * es
    R = max(1, min(max_sets, math.ceil(2 * MALL_BYTES / set_bytes)))
    keys = ("x", "delta", "lam", "Are", "theta", "Bm", "Cm", "D", "z")
    sets = []
    for r in range(R):
        w = si.scan3_inputs(B, L, D, N, dtype=wl["dtype"], seed=r)
        t = {k: si.to_torch(w[k], dev) for k in keys}
        t["y"] = torch.empty_like(t["x"])
        t["hf"] = torch.empty((B, D, N, 2), dtype=torch.float32, device=dev)
        sets.append(t)
    ws = torch.empty(max(ssa.ssm_scan3_workspace_size(B, L, D, N), 1), dtype=torch.uint8, device=dev)

    def call(t):
        ssa.ssm_scan3_fwd(t["x"], t["delta"], t["lam"], t["Are"], t["theta"], t["Bm"], t["Cm"], D=t["D"], z=t["z"],
                          y=t["y"], h_final=t["hf"], workspace=ws)

    nk = count_kernels(lambda: call(sets[0]))
    total_ms, ker = time_calls(call, sets, steps, warmup, nk)
    lat = latency(call, sets)
    ms = total_ms / steps
    kmean = ker.mean(axis=0)
    dom = int(np.argmax(kmean))
    upd = B * L * D * N
    alg = 5 * B * L * D * es + 2 * B * L * N * es + 2 * D * N * 4 + D * 4 + 2 * B * D * N * 4
    slots = SCAN3_FMA_OPS_PER_UPDATE + SCAN3_TRANS_PER_UPDATE * trans_cost
    achieved = slots * upd / (kmean[dom] * 1e-3) / 1e12
    peak = LANE_SLOTS_PER_S / 1e12
    return dict(workload=name, ms_per_step=ms, updates_per_s=upd / (ms * 1e-3), tokens_per_s=B * L / (ms * 1e-3),
                call_latency=lat, kernel_ms=[float(v) for v in kmean], hbm_gbs=alg / (ms * 1e-3) / 1e9,
                hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, sets=len(sets), alg_bytes=alg,
                roofline=dict(bound="alu", achieved=achieved, peak=peak, unit="Tslot/s", frac=achieved / peak,
                              slots_per_update=slots, traffic=committed_traffic("scan3", f"traffic_{name}.md"),
                              kernel="seg_final3 (dominant)"),
                alu=alu_figures(committed_valu("scan3", f"valu_{name}.md"), ["seg_agg3", "carry3", "seg_final3"],
                                kmean, ms, upd, trans_cost, one_pass=slots,
                                one_pass_note="11 FMA-class ops, one exp, one sin and one cos per update"))


# ------------------------------------------------------------------ scan backward
# Per state update, the final backward pass must issue: forward recompute v_mul
# (Delta*A), v_exp_f32, v_mul (u*B), v_fma (state), v_fma (C.h), v_mul (dv*h for dC);
# backward v_fma (adjoint), v_mul + v_exp_f32 (decay again), v_fma (a_t h_{t-1}), v_mul
# (q), v_fma x 3 (ddelta, dA, dx sums), v_mul (g*u for dB), v_mul (carry) -> 14 FMA-class
# ops and two v_exp_f32; plus the sums over the 64 channels of a wave for dB and dC, at
# least 2 x 63/64 adds -> 16 FMA-class ops and two exps per update.
BWD_FMA_OPS_PER_UPDATE = 16.0
BWD_EXPS_PER_UPDATE = 2.0


def scan_bwd_bench(name, wl, steps, warmup, dev, max_sets=8, trans_cost=DEFAULT_TRANS_COST):
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
    lat = latency(call, sets)
    ms = total_ms / steps
    kmean = ker.mean(axis=0)
    dom = int(np.argmax(kmean))
    upd = B * L * D * N
    # algorithmic bytes: read x, Delta, z, dy, B, C, A, D, dh_final; write dx, ddelta, dz,
    # dB, dC, dA, dD, dh0
    alg = 7 * B * L * D * es + 4 * B * L * N * es + 2 * (D * N + D) * 4 + 2 * B * D * N * 4
    tdom = kmean[dom] * 1e-3
    achieved = (BWD_FMA_OPS_PER_UPDATE + BWD_EXPS_PER_UPDATE * trans_cost) * upd / tdom / 1e12
    peak = LANE_SLOTS_PER_S / 1e12
    return dict(workload=name, ms_per_step=ms, updates_per_s=upd / (ms * 1e-3),
                tokens_per_s=B * L / (ms * 1e-3), call_latency=lat, kernel_ms=[float(v) for v in kmean],
                hbm_gbs=alg / (ms * 1e-3) / 1e9, hbm_frac=alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                sets=len(sets), alg_bytes=alg,
                roofline=dict(bound="alu", achieved=achieved, peak=peak, unit="Tslot/s", frac=achieved / peak,
                              traffic=committed_traffic("scan_bwd", f"traffic_{name}.md"),
                              kernel="bwd_final"),
                alu=alu_figures(committed_valu("scan_bwd", f"valu_{name}.md"), bwd_kernel_names(nk), kmean, ms,
                                upd, trans_cost, one_pass=BWD_FMA_OPS_PER_UPDATE + BWD_EXPS_PER_UPDATE * trans_cost,
                                one_pass_note="the final pass's 16 FMA-class ops and two exps per update"))


def bwd_kernel_names(nk):
    """The backward call's launches in order (N >= 32 adds the chunk-sum combine)."""
    base = ["bwd_aggregate", "bwd_carry_state", "bwd_carry_adjoint", "bwd_final"]
    tail = ["bwd_reduce_params", "bwd_reduce_rows"]
    if nk == 7:
        return base + ["bwd_combine"] + tail
    if nk == 6:
        return base + tail
    return [f"kernel{i}" for i in range(nk)]


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
    lat = latency(call, sets)
    warm = warm_ms(call, sets[0])
    ms = total_ms / steps
    kmean = ker.mean(axis=0)
    byt, fl = ssd_alg(wl)
    upd = B * L * H * P * N
    tdom = kmean[int(np.argmax(kmean))] * 1e-3
    return dict(workload=name, ms_per_step=ms, updates_per_s=upd / (ms * 1e-3),
                tokens_per_s=B * L / (ms * 1e-3), call_latency=lat, kernel_ms=[float(v) for v in kmean],
                hbm_gbs=byt / (ms * 1e-3) / 1e9, hbm_frac=byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                mfma_tflops=fl / (ms * 1e-3) / 1e12,
                mfma_frac=fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                roofline=dict(bound="hbm", achieved=byt / (ms * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              traffic=committed_traffic("ssd", f"ssd_kernels_{name[4:]}.md"),
                              kernel="whole call (three kernels)"),
                dominant_kernel_ms=tdom * 1e3, alg_bytes=byt, alg_flops=fl, warm_ms_per_step=warm)


def ssd_cpu_oracle(wl, heads=16):
    """The fp64 oracle's SSD in both forms, sequential (O2) and chunked at the
    workload's chunk length (O3), on one batch row and `heads` heads over the whole
    sequence, all host threads (one (batch, head) per thread)."""
    import oracle
    import ssm_inputs as si
    o = oracle.get()
    o.set_threads(len(os.sched_getaffinity(0)))
    L, H, P, N, Q = wl["L"], wl["H"], wl["P"], wl["N"], wl["chunk"]
    h = min(heads, H)
    w = si.ssd_inputs(1, L, h, P, N, seed=0)
    f = {k: si.to_f64(w[k]) for k in ("x", "delta", "Bm", "Cm", "A")}
    upd = L * h * P * N
    out = {}
    for form, fn in (("sequential", lambda: o.ssd_seq(f["x"], f["delta"], f["A"], f["Bm"], f["Cm"])),
                     ("chunked", lambda: o.ssd_chunked(f["x"], f["delta"], f["A"], f["Bm"], f["Cm"], chunk=Q))):
        t0 = time.perf_counter()
        fn()
        el = time.perf_counter() - t0
        out[form] = dict(value=upd / el, unit="state updates/s", seconds=el)
    out.update(cores=o.get_threads(), kind="oracle", sample=f"B=1, L={L}, {h} of {H} heads, P={P}, N={N}, chunk {Q}")
    return out


def copy_gbs(dev, reps=5):
    """This library's plain 1 GiB device copy (ssm_diag_copy), GB/s moved (read + write)."""
    import torch
    import selective_scan_amd as ssa
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ssa.ssm_diag_copy(src, dst)
    sync()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        ssa.ssm_diag_copy(src, dst)
    t1.record()
    sync()
    ms = t0.elapsed_time(t1) / reps
    nb = 2 * src.numel() * 4
    return dict(gbs=nb / (ms * 1e-3) / 1e9, frac=nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, ms=ms, bytes=nb,
                kernel="copy16 (ssm_diag_copy), 1 GiB")


# ------------------------------------------------------------------ decode
def step_bench(wl, dev, reps=3, only=None):
    """The decode workload: `steps` in-place steps, stream-launched and HIP-graph
    replayed (state MALL-resident), then the cold multi-layer variant and the
    streaming floor. only="hot" / "cold": just that graph-replayed variant (for
    counter runs that must not mix the two)."""
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

    step1 = (lambda stv, s_: ssa.ssm_step(stv, tok["x"][s_], tok["delta"][s_], A, tok["Bm"][s_], tok["Cm"][s_],
                                          D=Dk, z=tok["z"][s_], y=y[s_]))
    if only == "cold":
        cold = cold_decode(step1, st0, steps)
        return dict(workload="step_bf16_B64_D3072_N16_x1000", only="cold", cold_ms_per_step=cold["ms"],
                    layers=cold["layers"])
    times = []
    if only is None:
        run()
        sync()
        for _ in range(reps):
            st.copy_(st0)
            sync()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            sync()
            times.append(e0.elapsed_time(e1))
    # HIP-graph replay of the same launches
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
    if only == "hot":
        return dict(workload="step_bf16_B64_D3072_N16_x1000", only="hot",
                    hot_ms_per_step=float(np.median(gtimes)) / steps)
    es = 2 if wl["dtype"] == "bf16" else 4
    alg = 2 * B * D * N * 4 + 4 * B * D * es + 2 * B * N * es + (D * N + D) * 4
    med = float(np.median(times)) / steps
    gmed = float(np.median(gtimes)) / steps
    cold = cold_decode(step1, st0, steps)
    return dict(workload="step_bf16_B64_D3072_N16_x1000", ms_per_step_stream=med,
                traffic=committed_traffic("step", "traffic_step_bf16_B64_D3072_N16.md"), alg_bytes_per_step=alg,
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


def step3_bench(wl, dev, reps=3, only=None):
    """The Mamba-3 decode workload: `steps` in-place steps of ssm_step3, each given the
    previous token, stream-launched and HIP-graph replayed (state MALL-resident), then
    the cold multi-layer variant and the streaming floor. only="hot" / "cold" as for
    step_bench."""
    import torch
    import selective_scan_amd as ssa
    import ssm_inputs as si
    name = "step3_bf16_B64_D3072_N16_x200"
    B, D, N, steps = wl["B"], wl["D"], wl["N"], wl["steps"]
    w = si.scan3_inputs(B, steps, D, N, dtype=wl["dtype"], seed=0, with_h0=True, with_prev=True)
    # token-major copies, so that token s is a contiguous, aligned [B, ...] slice
    tok = {k: si.to_torch(np.ascontiguousarray(np.swapaxes(w[k], 0, 1)), dev)
           for k in ("x", "delta", "lam", "z", "Bm", "Cm")}
    Are, th = torch.from_numpy(w["Are"]).to(dev), torch.from_numpy(w["theta"]).to(dev)
    Dk = torch.from_numpy(w["D"]).to(dev)
    xp0, bp0 = si.to_torch(w["x_prev"], dev), si.to_torch(w["B_prev"], dev)
    st0 = torch.from_numpy(w["h0"]).to(dev)
    st = st0.clone()
    y = torch.empty((steps, B, D), dtype=tok["x"].dtype, device=dev)

    def step1(stv, s_):
        xp, bp = (xp0, bp0) if s_ == 0 else (tok["x"][s_ - 1], tok["Bm"][s_ - 1])
        ssa.ssm_step3(stv, tok["x"][s_], tok["delta"][s_], tok["lam"][s_], Are, th, tok["Bm"][s_], tok["Cm"][s_],
                      D=Dk, z=tok["z"][s_], x_prev=xp, B_prev=bp, y=y[s_])

    def run():
        for s_ in range(steps):
            step1(st, s_)

    if only == "cold":
        cold = cold_decode(step1, st0, steps)
        return dict(workload=name, only="cold", cold_ms_per_step=cold["ms"], layers=cold["layers"])
    times = []
    if only is None:
        run()
        sync()
        for _ in range(reps):
            st.copy_(st0)
            sync()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            sync()
            times.append(e0.elapsed_time(e1))
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
    if only == "hot":
        return dict(workload=name, only="hot", hot_ms_per_step=float(np.median(gtimes)) / steps)
    es = 2 if wl["dtype"] == "bf16" else 4
    # complex state read and written; x, Delta, lam, z, x_prev read and y written; B, C,
    # B_prev rows; Are, theta and D
    alg = 2 * B * D * N * 8 + 6 * B * D * es + 3 * B * N * es + (2 * D * N + D) * 4
    med = float(np.median(times)) / steps
    gmed = float(np.median(gtimes)) / steps
    cold = cold_decode(step1, st0, steps)
    return dict(workload=name, ms_per_step_stream=med,
                traffic=committed_traffic("step3", "traffic_step3_bf16_B64_D3072_N16.md"), alg_bytes_per_step=alg,
                ms_per_step_graph=gmed, updates_per_s_graph=B * D * N / (gmed * 1e-3),
                tokens_per_s_graph=B / (gmed * 1e-3), hbm_gbs_graph=alg / (gmed * 1e-3) / 1e9,
                note="complex state (%.1f MB) stays resident in the 256 MB MALL across in-place steps"
                     % (st0.numel() * 4 / 1e6),
                cold=dict(layers=cold["layers"], ms_per_step_graph=cold["ms"],
                          hbm_gbs_graph=alg / (cold["ms"] * 1e-3) / 1e9,
                          hbm_frac=alg / (cold["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          note="step s updates the state of layer s mod layers: the states "
                               "(%d x %.1f MB) exceed the MALL, so each step streams its state from HBM"
                               % (cold["layers"], st0.numel() * 4 / 1e6)),
                streaming_floor=streaming_floor(st0, steps))


def streaming_floor(st0, steps, reps=3):
    """Context for a decode step: this library's in-place streaming kernel
    (ssm_diag_stream_scale: every 16-byte load of a lane issued before its first
    store, one launch per step) on a tensor of the state's size, graph-replayed
    `steps` times on one tensor (MALL-resident) and rotating over tensors adding up
    to more than the MALL. What one launch per step reaches by pure streaming."""
    import torch
    import selective_scan_amd as ssa
    st = st0.clone()
    g = torch.cuda.CUDAGraph()
    sync()
    s_ = torch.cuda.Stream()
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            for _ in range(steps):
                ssa.ssm_diag_stream_scale(st, 0.999)
    sync()
    hot = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        sync()
        hot.append(e0.elapsed_time(e1) / steps)
    cold = cold_decode(lambda stv, s_: ssa.ssm_diag_stream_scale(stv, 0.999), st0, steps, reps=reps)
    nb = 2 * st0.numel() * 4
    return dict(ms_per_step_hot=float(np.median(hot)), ms_per_step_cold=cold["ms"], bytes_per_step=nb,
                hbm_frac_cold=nb / (cold["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                note="ssm_diag_stream_scale (this library's in-place streaming kernel) on a tensor of the "
                     "state's size, graph-replayed like the steps: reads and writes the state only")


def valu_rates(dev, blocks=8192, iters=2048):
    """The VALU issue-rate probes: exp-only, fma-only, 1:3, sin-only and cos-only
    chains, full occupancy."""
    import torch
    import selective_scan_amd as ssa
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    res = {}
    for mode, nm in ((0, "exp"), (1, "fma"), (2, "exp1_fma3"), (3, "sin"), (4, "cos")):
        ssa.ssm_diag_valu_rate(mode, out, 16)
        sync()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ops = ssa.ssm_diag_valu_rate(mode, out, iters)
        e1.record()
        sync()
        ms = e0.elapsed_time(e1)
        res[nm] = dict(ops_per_s=ops / (ms * 1e-3), ms=ms, ops=ops)
    fma, ex = res["fma"]["ops_per_s"], res["exp"]["ops_per_s"]
    mix = res["exp1_fma3"]["ops_per_s"]
    res["exp_cost_in_fma_slots"] = fma / ex
    res["sin_cost_in_fma_slots"] = fma / res["sin"]["ops_per_s"]
    res["cos_cost_in_fma_slots"] = fma / res["cos"]["ops_per_s"]
    # if exp and fma shared one issue port with costs c_e and 1, a 1:3 mix would run at
    # 4 / (c_e + 3) of the fma rate; co-issue would show as a faster mix
    res["mix_predicted_no_coissue_ops_per_s"] = 4.0 * fma / (fma / ex + 3.0)
    res["mix_measured_over_predicted"] = mix / res["mix_predicted_no_coissue_ops_per_s"]
    res["fma_frac_of_lane_peak"] = fma / LANE_SLOTS_PER_S
    res["note"] = ("lane ops/s of ssm_diag_valu_rate: 8 independent chains per lane, %d lanes; the lane-slot "
                   "peak is 256 CU x 128 lane-ops per clock (4 SIMDs, a wave64 instruction every 2 clocks) "
                   "x 2.4 GHz = %.1f T/s" % (blocks * 256, LANE_SLOTS_PER_S / 1e12))
    return res


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


def ssd_step_bench(wl, dev, reps=3, only=None):
    """Mamba-2 decode: `steps` in-place steps launched on a stream, then the same
    steps replayed from a HIP graph; per-step time and algorithmic bytes/s.
    only="hot" / "cold": just that graph-replayed variant (for counter runs)."""
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

    step1 = (lambda stv, s_: ssa.ssm_ssd_step(stv, tok["x"][s_], tok["delta"][s_], A, tok["Bm"][s_],
                                              tok["Cm"][s_], D=Dk, z=tok["z"][s_], y=y[s_]))
    if only == "cold":
        cold = cold_decode(step1, st0, steps)
        return dict(workload="ssd_step_bf16_B64_H24_P64_N128_x200", only="cold", cold_ms_per_step=cold["ms"],
                    layers=cold["layers"])
    ms_stream = None
    if only is None:
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
    if only == "hot":
        return dict(workload="ssd_step_bf16_B64_H24_P64_N128_x200", only="hot", hot_ms_per_step=ms_graph)
    es = 2 if wl["dtype"] == "bf16" else 4
    alg = 2 * B * H * N * P * 4 + 3 * B * H * P * es + B * H * es + 2 * B * N * es + 2 * H * 4
    cold = cold_decode(step1, st0, steps)
    return dict(workload="ssd_step_bf16_B64_H24_P64_N128_x200", ms_per_step_stream=ms_stream,
                traffic=committed_traffic("ssd_step", "traffic_ssd_step_bf16_B64_H24_P64_N128.md"),
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


def scan_summary(r):
    keys = ("workload", "ms_per_step", "updates_per_s", "tokens_per_s", "call_latency", "hbm_gbs", "hbm_frac",
            "kernel_ms", "roofline", "alu", "warm_ms_per_step")
    return {k: r[k] for k in keys if k in r}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-other", action="store_true")
    ap.add_argument("--other", default=None,
                    help="only run this one workload of the other paths (a scan_*, scan_bwd_*, scan_zoh_*, ssd_*, "
                         "step_*, ssd_step_* or step3_* name) and print it")
    ap.add_argument("--decode-pass", choices=("hot", "cold"), default=None,
                    help="with --other step_*/ssd_step_*/step3_*: run only the graph-replayed hot or cold variant")
    ap.add_argument("--valu-rates", action="store_true",
                    help="only run the VALU issue-rate probes (exp, fma, 1:3 mix) and print them")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (ssm_diag_copy) 5 times (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the selective scan here has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import ssm_inputs as si
    import selective_scan_amd as ssa
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            ssa.ssm_diag_copy(src, dst)
        sync()
        print(json.dumps({"calibrate_copy_bytes_read": src.numel() * 4, "calibrate_copy_bytes_written": dst.numel() * 4,
                          "launches": 5, "kernel": "copy16 (ssm_diag_copy)"}))
        return
    if args.valu_rates:
        print(json.dumps(valu_rates(dev)))
        return
    if args.other:
        wl = si.WORKLOADS[args.other]
        if wl["kind"] == "scan_bwd":
            r = scan_bwd_bench(args.other, wl, args.steps, args.warmup, dev)
        elif wl["kind"] == "scan_var":
            r = scan_var_bench(args.other, wl, args.steps, args.warmup, dev)
        elif wl["kind"] == "scan3":
            r = scan3_bench(args.other, wl, args.steps, args.warmup, dev)
        elif wl["kind"] == "ssd":
            r = ssd_bench(args.other, wl, args.steps, args.warmup, dev)
        elif wl["kind"] == "scan":
            r = scan_summary(scan_bench(args.other, wl, args.steps, args.warmup, dev)[0])
        elif wl["kind"] == "step":
            r = step_bench(wl, dev, only=args.decode_pass)
        elif wl["kind"] == "ssd_step":
            r = ssd_step_bench(wl, dev, only=args.decode_pass)
        elif wl["kind"] == "step3":
            r = step3_bench(wl, dev, only=args.decode_pass)
        else:
            raise SystemExit(f"--other takes a scan_*, scan_bwd_*, scan_zoh_* or ssd_* workload, not {args.other}")
        print(json.dumps(r))
        return
    wl = si.WORKLOADS[args.workload]
    assert wl["kind"] == "scan", "the headline bench line is a scan workload"
    rates = valu_rates(dev)
    trans_cost = rates["exp_cost_in_fma_slots"]
    res, w0 = scan_bench(args.workload, wl, args.steps, args.warmup, dev, trans_cost=trans_cost)
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
        "device": device_info(dev),
        "tokens_per_s": res["tokens_per_s"],
        "hbm_gbs": res["hbm_gbs"],
        "hbm_frac": res["hbm_frac"],
        "call_latency": res["call_latency"],
        "kernel_ms": res["kernel_ms"],
        "roofline": res["roofline"],
        "alu": res["alu"],
        "context": dict(PAGE_CONTEXT, this_run=dict(
            hbm_frac_call=res["hbm_frac"], updates_per_s=res["updates_per_s"],
            note="this line's own HBM fraction, beside the pages' 0.01-0.15 % for per-timestep Python loops")),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = scan_cpu_baseline(wl, w0)
    del w0
    if not args.no_other:
        other = {"valu_rates": rates}
        for nm in ("scan_f32_B1_L256_D64_N16", "scan_bf16_B1_L4096_D1536_N16", "scan_bf16_B1_L4096_D1536_N64",
                   "scan_bf16_B1_L4096_D1536_N128", "scan_bf16_B1_L4096_D1536_N256"):
            if nm == args.workload:
                continue
            r3, _ = scan_bench(nm, si.WORKLOADS[nm], steps=20, warmup=3, dev=dev, trans_cost=trans_cost)
            other[nm] = scan_summary(r3)
        other["scan_f32_B1_L256_D64_N16"]["latency_us"] = {
            k: v * 1e3 for k, v in other["scan_f32_B1_L256_D64_N16"]["call_latency"].items() if k.endswith("_ms")}
        for nm in ("scan_zoh_softplus_bf16_B1_L4096_D1536_N16", "scan_zoh_softplus_bf16_B1_L4096_D1536_N64"):
            other[nm] = scan_var_bench(nm, si.WORKLOADS[nm], steps=20, warmup=3, dev=dev, trans_cost=trans_cost)
        other["scan3_bf16_B1_L4096_D1536_N16"] = scan3_bench(
            "scan3_bf16_B1_L4096_D1536_N16", si.WORKLOADS["scan3_bf16_B1_L4096_D1536_N16"], steps=20, warmup=3,
            dev=dev, trans_cost=trans_cost)
        for nm in ("scan_bwd_bf16_B1_L4096_D1536_N16", "scan_bwd_bf16_B8_L32768_D512_N16",
                   "scan_bwd_bf16_B1_L4096_D1536_N64"):
            other[nm] = scan_bwd_bench(nm, si.WORKLOADS[nm], steps=10 if si.WORKLOADS[nm]["L"] <= 4096 else 3,
                                       warmup=2, dev=dev, trans_cost=trans_cost)
        for nm in ("ssd_bf16_B4_L8192_H24_P64_N128_Q256", "ssd_bf16_B4_L8192_H24_P64_N128_Q64",
                   "ssd_bf16_B4_L8000_H24_P64_N128_Q256"):
            other[nm] = ssd_bench(nm, si.WORKLOADS[nm], steps=10, warmup=3, dev=dev)
            if not args.no_cpu and nm.endswith("Q256") and "L8192" in nm:
                other[nm]["cpu_oracle"] = ssd_cpu_oracle(si.WORKLOADS[nm])
        other["copy"] = copy_gbs(dev)
        other["decode"] = step_bench(si.WORKLOADS["step_bf16_B64_D3072_N16_x1000"], dev)
        other["ssd_decode"] = ssd_step_bench(si.WORKLOADS["ssd_step_bf16_B64_H24_P64_N128_x200"], dev)
        other["mamba3_decode"] = step3_bench(si.WORKLOADS["step3_bf16_B64_D3072_N16_x200"], dev)
        out["other_paths"] = other
    print(json.dumps(out))


if __name__ == "__main__":
    main()
