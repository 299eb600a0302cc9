"""Compile the gfx950 HIP library ``libssm_scan.so`` in-tree with hipcc.

    python -m selective_scan_amd.build            # build (always recompiles)
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssm_scan.so")

SOURCES = ["api.cpp", "scan_fwd.hip", "scan_var.hip", "scan3.hip", "step3.hip", "scan_noalloc.hip", "scan_bwd.hip",
           "step.hip", "ssd_fwd.hip", "ssd_step.hip", "diag.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU forms are switched off for every device compile.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-I", INCLUDE, "-I", CSRC]


def _compile(src, obj):
    path = os.path.join(CSRC, src)
    flags = COMMON + (DEVICE_FLAGS if src.endswith(".hip") else [])
    cmd = [HIPCC, *flags, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    return err


def build(verbose=False):
    """Compile every source and link ``libssm_scan.so``; returns its path."""
    with tempfile.TemporaryDirectory(prefix="ssm_build_") as tmp:
        objs = [os.path.join(tmp, s.replace(".", "_") + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
            msgs = list(ex.map(_compile, SOURCES, objs))
        if verbose:
            for s, m in zip(SOURCES, msgs):
                if m:
                    sys.stderr.write(f"[{s}] {m}\n")
        out_tmp = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + " ".join(cmd) + "\n" + r.stderr)
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
