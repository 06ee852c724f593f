"""Build libssd.so (HIP, gfx950) in-tree with hipcc.

``python -m ssd_chunked_scan_03_amd.build`` compiles every ``csrc/*.hip`` unit in
parallel and links them into ``ssd_chunked_scan_03_amd/libssd.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssd.so")
PEAK_SRC = os.path.join(PKG, "peak", "peak.hip")
PEAK_LIB = os.path.join(PKG, "libssd_peak.so")  # measurement kernels for the benchmark only
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    t0 = time.time()
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, LIB)
    # the benchmark's measured denominators (streaming copy, matrix-core loop)
    tmp = PEAK_LIB + ".tmp"
    r = subprocess.run([HIPCC, *CFLAGS, "-shared", PEAK_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PEAK_SRC}:\n{r.stderr[-8000:]}")
    os.replace(tmp, PEAK_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} units in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
