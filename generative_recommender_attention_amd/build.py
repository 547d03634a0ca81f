"""Build ``libhstu.so`` for gfx950 with hipcc (ahead of time, in-tree), and its
debug variant ``libhstu_debug.so`` (-DHSTU_DEBUG: bounds tests on the kernels'
global indices, read back with hstu_debug_take).

Usage:  python -m generative_recommender_attention_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "libhstu")
LIB_PATH = os.path.join(PKG, "libhstu.so")
DEBUG_BUILD_DIR = os.path.join(ROOT, "_build", "libhstu_debug")
DEBUG_LIB_PATH = os.path.join(PKG, "libhstu_debug.so")

SOURCES = ["hstu_api.cpp", "hstu_fwd.hip", "hstu_bwd.hip", "lmsd.hip", "clock.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# Per-source scheduler choice: the backward kernels run faster when the machine
# scheduler favours instruction-level parallelism over register pressure (they
# still fit their register budgets without spills); the forward does not.
FILE_FLAGS = {"hstu_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libhstu")
    return path


def compile_flags():
    return ["-std=c++17", "-O3", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS


def _compile(job) -> str:
    src, debug = job
    obj = os.path.join(DEBUG_BUILD_DIR if debug else BUILD_DIR, os.path.basename(src) + ".o")
    extra = ["-DHSTU_DEBUG"] if debug else []
    cmd = [hipcc(), *compile_flags(), *extra, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass reports the device-only feature flag as unknown; drop that line only.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = True, debug: bool = True) -> str:
    """Compile every source and link ``libhstu.so`` next to this file (and, with
    ``debug``, ``libhstu_debug.so``)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(DEBUG_BUILD_DIR, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + ([(s, True) for s in SOURCES] if debug else [])
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    if debug:
        _link(objs[len(SOURCES):], DEBUG_LIB_PATH)
        if verbose:
            print(f"built {DEBUG_LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
