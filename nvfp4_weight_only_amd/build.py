"""Build libnvfp4.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m nvfp4_weight_only_amd.build

Flags: gfx950 only; -O3 without fast-math; no FP contraction (the quantizer
and the dequantizer round exactly where the format says); packed FP32 VALU
instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libnvfp4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["nvfp4_abi.hip", "quant_kernels.hip", "gemv.hip", "gemm.hip", "skinny.hip", "prefill.hip", "grouped.hip", "kv_gather.hip", "mxfp4.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnvfp4.so)")


def compile_flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link libnvfp4.so next to this file; returns its path."""
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    # -z defs: every symbol the library uses must resolve at link time (a missing
    # launcher would otherwise surface only when the library is loaded).
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
