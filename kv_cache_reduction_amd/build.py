"""Builds libslim.so in-tree for gfx950 with hipcc.

    python kv_cache_reduction_amd/build.py          # always recompiles

Objects go to ``_build/`` at the repository root; the library lands next to
this file.  HIP sources are compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libslim.so")

HIP_SOURCES = ["api.hip", "attend_bf16.hip", "attend_f32.hip", "finish.hip", "mha_kv.hip",
               "multi.hip", "prefill.hip", "probe.hip", "step.hip"]
CPP_SOURCES = ["wkv_host.cpp"]
# The bf16 attend and many-query kernels never see NaN in the rows they read
# (they only take maxima of finite scores and -inf); without this flag every
# fmaxf first quiets possible signalling NaNs with an extra instruction.
EXTRA_FLAGS = {"attend_bf16.hip": ["-fno-honor-nans"], "multi.hip": ["-fno-honor-nans"]}
ARCH = os.environ.get("SLIM_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _hip_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD, s.replace(".hip", ".o"))
        jobs.append([hipcc, *_hip_flags(), *EXTRA_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", obj])
    for s in CPP_SOURCES:
        obj = os.path.join(BUILD, s.replace(".cpp", ".o"))
        jobs.append(["g++", "-O3", "-std=c++17", "-fPIC", "-march=x86-64-v3", "-Wall",
                     "-c", os.path.join(CSRC, s), "-o", obj])
    nproc = max(1, min(16, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(nproc) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                sys.stderr.write(r.stdout + r.stderr)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, "-lpthread"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
