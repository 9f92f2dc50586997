"""Build libfva.so in-tree with hipcc for gfx950.

Usage: python -m block_sparse_spatiotemporal_amd.build   (or call build()).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfva.so")
SOURCES = ["plan.cpp", "permute.hip", "select.hip", "attention.hip", "backward.hip"]
# The attention kernels take row maxima of matrix-core results, which in IEEE
# mode cost a NaN-quieting max per operand; they compute no NaN from finite
# inputs, so that file is built without IEEE mode and without NaN semantics.
EXTRA = {"attention.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libfva.so next to this file."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              "-Wall", "-Wno-unused-function"]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [hipcc()] + common + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        cmd[1:1] = ["-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-ffp-contract=fast"]
        if verbose:
            print(" ".join(cmd), flush=True)
        cmds.append(cmd)
        objs.append(obj)
    # the sources compile independently: run them side by side
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "4"))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for r in list(ex.map(lambda c: subprocess.run(c), cmds)):
            if r.returncode != 0:
                raise subprocess.CalledProcessError(r.returncode, r.args)
    tmp = LIB + ".tmp"
    subprocess.run([hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
