"""Ahead-of-time build of libak.so for gfx950 (hipcc for the kernels and the C
ABI, the host C++ compiler for the planner).  Run as a script or call build()."""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libak.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]
# per-source code generation options
FILE_FLAGS = {}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hip, cpp = sources()
    jobs = []
    for f in hip:
        obj = os.path.join(BUILD_DIR, f + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *FILE_FLAGS.get(f, []), "-c", os.path.join(CSRC, f), "-o", obj])
    for f in cpp:
        obj = os.path.join(BUILD_DIR, f + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, f), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for r in ex.map(_run, jobs):
            if verbose and r.stderr:
                print(r.stderr, file=sys.stderr)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp])
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
