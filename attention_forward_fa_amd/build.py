"""Build ``libfa_fwd.so`` (the C-ABI library) in-tree for gfx950.

    python -m attention_forward_fa_amd.build

The host planner (phase 1) is plain C++ and is compiled with g++; the kernels
and the phase-2 launcher are HIP, compiled with hipcc for gfx950.  Objects go
to ``_build/`` at the repository root; the library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa_fwd.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled: the compiler must not form them.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]

HIP_SOURCES = ["fa_launch.hip", "fa_mfma_bf16.hip", "fa_mfma_f16.hip", "fa_generic.hip", "fa_merge.hip"]
# Extra flags per source.  The matrix-core kernel never produces NaN from
# finite inputs, so max needs no NaN canonicalisation.
PER_SOURCE_FLAGS = {"fa_mfma_bf16.hip": ["-fno-honor-nans"], "fa_mfma_f16.hip": ["-fno-honor-nans"]}
CXX_SOURCES = ["fa_plan.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the library.  Always rebuilds; a failed
    build leaves no library behind (never a stale one)."""
    os.makedirs(BUILD, exist_ok=True)
    if os.path.exists(LIB):
        os.remove(LIB)
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, *PER_SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
