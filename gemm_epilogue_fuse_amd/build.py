"""Ahead-of-time build of libfuse.so for gfx950 with hipcc.

``python -m gemm_epilogue_fuse_amd.build`` (or ``build()``) compiles the HIP
kernels and the C-ABI host code in ``csrc/`` into ``libfuse.so`` next to this
file.  Compilation happens on any machine with ROCm; no GPU is needed.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libfuse.so")
ARCH = "gfx950"

# One unit per kernel family, so the units compile in parallel.
SOURCES = ["gemm_fused.hip", "k_dma_square.hip", "k_dma_wide.hip", "k_dma_pro.hip", "k_reg.hip", "k_small.hip",
           "fuse_api.cpp"]
HEADERS = ["launch.h", "kernels.h"]

# Packed-fp32 VALU forms are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: ROCm is required to build libfuse")


def build(verbose: bool = False) -> str:
    """Compile every source and link libfuse.so (always recompiles)."""
    cc = hipcc()
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I" + INCLUDE, "-I" + CSRC,
               "-Wall", "-Wno-unused-function"]
        if src.endswith(".hip"):
            cmd += ["-x", "hip"] + DEVICE_FLAGS
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        _, err = pr.communicate()
        if pr.returncode != 0:
            failed.append("hipcc failed on %s:\n%s" % (src, err))
    if failed:
        raise RuntimeError("\n".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
