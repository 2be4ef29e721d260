"""Build the HIP relation-KL library (liblard.so) in-tree for gfx950.

    python -m attention_relation_distillation_amd.build

Compiles the HIP kernels with hipcc for gfx950 (packed-fp32 instructions disabled), the
host-side C ABI with g++, and links them into attention_relation_distillation_amd/liblard.so.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblard.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++20", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, extra_hip_flags=()) -> str:
    """Compile and link liblard.so; returns its path.  Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    for name in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, name)
        obj = os.path.join(BUILD, name + ".o")
        if name.endswith(".hip"):
            jobs.append([HIPCC, *HIP_FLAGS, *extra_hip_flags, "-c", src, "-o", obj])
        elif name.endswith(".cpp"):
            jobs.append([shutil.which("g++") or "g++", *CXX_FLAGS, "-c", src, "-o", obj])
        else:
            continue
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r, cmd in zip(ex.map(_run, jobs), jobs):
            if verbose:
                print(" ".join(cmd))
                if r.stderr.strip():
                    print(r.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
