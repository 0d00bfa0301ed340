"""Builds libikbo.so in-tree with hipcc for gfx950.

    python -m broadcast_free_target_amd._build

Each source compiles to an object under ``_build/`` (in parallel), then one
link produces ``broadcast_free_target_amd/libikbo.so``.  The library is
always rebuilt when this runs.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libikbo.so")

SOURCES = ("ikbo_plan.cpp", "ikbo_kernels.hip", "ikbo_lce.hip", "ikbo_bwd.hip", "ikbo_mx.hip", "ikbo_api.hip",
           "ikbo_api_lce.hip", "ikbo_api_bwd.hip", "ikbo_api_mx.hip", "ikbo_api_noalloc.hip")
ARCH = os.environ.get("IKBO_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are disabled for all device code.
HIP_FLAGS = [
    "-O3", "-std=c++20", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libikbo.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(BUILD, s.rsplit(".", 1)[0] + ".o")
        lang = ["-x", "hip"] if s.endswith(".hip") else []
        cmds.append([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, *lang, "-c", src, "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
