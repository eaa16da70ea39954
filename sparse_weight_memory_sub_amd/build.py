"""Build the gfx950 HIP library ``libfwpkm.so`` in-tree with hipcc.

Usage: ``python -m sparse_weight_memory_sub_amd.build`` (or ``build()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfwpkm.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["fwpkm_api.cpp", "k_score.hip", "k_gather.hip", "k_sort.hip", "k_scatter.hip", "k_addr.hip",
           "k_usage.hip", "k_backward.hip"]

ARCH = os.environ.get("FWPKM_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfwpkm.so)")


def _compile(src: str, hipcc: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


PROBE_SRC = os.path.join(HERE, "probe", "rows_probe.hip")
PROBE_OUT = os.path.join(HERE, "probe", "libfwpkm_probe.so")


def build_probe(hipcc: str) -> str:
    """The measurement library of bench.py --ceiling (not part of the layer)."""
    tmp = PROBE_OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc, *FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for rows_probe.hip:\n" + r.stderr)
    os.replace(tmp, PROBE_OUT)
    return PROBE_OUT


def build(verbose: bool = True) -> str:
    """Compile every HIP source for gfx950 and link libfwpkm.so (always
    rebuilds), and the measurement library of bench.py --ceiling."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        probe = ex.submit(build_probe, hipcc)
        objs = list(ex.map(lambda s: _compile(s, hipcc), SOURCES))
        probe.result()
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
