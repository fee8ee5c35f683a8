"""Compile the gfx950 library: hipcc -> varlen_prefill_amd/_build/librp.so.

Usage: python -m varlen_prefill_amd.build   (or __graft_entry__.build()).
Cross-compiles without a GPU.  Only gfx950 code objects are produced.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(BUILD, "librp.so")
INCLUDE = os.path.join(ROOT, "include")

# (source, object, extra flags): the tile kernel source is built twice, once
# for the plain tile kernels and once for the instances that also run fold
# items (in-workgroup chunk folding)
SOURCES = [
    ("rp_kernels.hip", "rp_kernels.o", []),
    ("rp_kernels.hip", "rp_kernels_fold.o", ["-DRP_TILE_FOLD=1"]),
    ("rp_state_merge.hip", "rp_state_merge.o", []),
    ("rp_noalloc.hip", "rp_noalloc.o", []),
    ("rp_plan.cpp", "rp_plan.o", []),
    ("rp_api.cpp", "rp_api.o", []),
]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 VALU forms are disabled for every HIP compile
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs, procs = [], []
    # the objects compile in parallel (the two tile-kernel objects dominate)
    for src, obj_name, extra in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, obj_name)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ([hipcc()] + HIPCC_FLAGS + extra + ["-I", INCLUDE, "-I", CSRC] + lang +
               ["-c", path, "-o", obj])
        if verbose:
            print(" ".join(cmd))
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    failed = []
    for src, proc in procs:
        out, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out)
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
