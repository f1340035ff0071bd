"""Builds ``libtokenweave.so`` in-tree for gfx950.

Host C++ (validation, planner) is compiled with g++; the kernels with hipcc
for gfx950 only.  Every HIP compile carries ``-Xclang -target-feature
-Xclang -packed-fp32-ops`` so that the compiler never emits packed float32
instructions.  Objects go to ``_build/`` at the repo root; the library lands
next to this file, where the binding loads it.

Usage: ``python -m reduce_rmsnorm_amd.build`` (or ``build()`` from Python).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libtokenweave.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]
# Host C++ uses the HIP runtime API only (pointer queries), through its C headers.
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
             "-I/opt/rocm/include"]

HOST_SOURCES = ["api.cpp", "split_plan.cpp"]
HIP_SOURCES = ["fused_reduce_rmsnorm.hip", "unfused.hip"]
# Per-source flags.  The fused one-row kernel takes its first three arguments
# (first tensor, first row, row length), the comparator's reduce kernel its
# first two (first tensor, row length), as scalars for the hardware to preload
# into SGPRs at wave launch, so a wave's first load need not wait for the
# argument block.
HIP_SOURCE_FLAGS = {"fused_reduce_rmsnorm.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=3"],
                    "unfused.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=2"]}
# The compiler's per-kernel resource report (registers, scratch, occupancy) of
# each kernel source, kept next to its object for the spill checks of the
# tests.
RESOURCE_FLAGS = ["-Rpass-analysis=kernel-resource-usage"]


def resource_report(src: str) -> str:
    return os.path.join(BUILD, src + ".resources.txt")
# Measurement-only bandwidth probes (bench.py --ceiling, counter calibration),
# built into a library of their own so the fused library carries none of them.
PROBE_SOURCE = "bw_probe.hip"
PROBE_LIB_PATH = os.path.join(PKG, "libtw_bwprobe.so")


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP extension cannot be built")


def _run_all(cmds, logs=None):
    """Runs the commands in parallel.  A command whose index has a path in
    ``logs`` writes its output there (the resource-usage remarks) instead of
    to stderr."""
    logs = logs or {}
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
             for c in cmds]
    failed = []
    for i, (c, p) in enumerate(procs):
        out, _ = p.communicate()
        # hipcc's host pass does not know the packed-fp32 target feature; harmless.
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln
                 and "is not a recognized feature for this target" not in ln]
        if i in logs:
            with open(logs[i], "w") as f:
                f.write("\n".join(lines) + "\n")
            lines = [ln for ln in lines if "error" in ln] if p.returncode != 0 else []
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
        if p.returncode != 0:
            failed.append(" ".join(c))
    if failed:
        raise RuntimeError("build failed:\n  " + "\n  ".join(failed))


def build(verbose: bool = False) -> str:
    """Compile and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs, cmds = [], []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *CXX_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    logs = {}
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        logs[len(cmds)] = resource_report(src)
        cmds.append([hipcc, *HIP_FLAGS, *HIP_SOURCE_FLAGS.get(src, []), *RESOURCE_FLAGS, "-I",
                     INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    if verbose:
        for c in cmds:
            print(" ".join(c))
    probe_obj = os.path.join(BUILD, PROBE_SOURCE + ".o")
    cmds.append([hipcc, *HIP_FLAGS, "-I", CSRC, "-c", os.path.join(CSRC, PROBE_SOURCE), "-o",
                 probe_obj])
    if verbose:
        print(" ".join(cmds[-1]))
    _run_all(cmds, logs)
    tmp, ptmp = LIB_PATH + ".tmp", PROBE_LIB_PATH + ".tmp"
    _run_all([[hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs],
              [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", ptmp, probe_obj]])
    os.replace(tmp, LIB_PATH)
    os.replace(ptmp, PROBE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
