"""Build libnvfp4.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m nvfp4_weight_only_amd.build

Flags: gfx950 only; -O3 without fast-math; no FP contraction (the quantizer
and the dequantizer round exactly where the format says); packed FP32 VALU
instructions disabled.
"""
from __future__ import annotations

import concurrent.futures
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
SOURCES = ["nvfp4_abi.hip", "quant_kernels.hip", "gemv.hip", "gemm.hip", "skinny.hip", "small_m.hip", "prefill.hip", "grouped.hip", "kv_gather.hip", "mxfp4.hip", "stream.hip"]


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
    objs = [os.path.join(objdir, src + ".o") for src in SOURCES]
    cmds = [[cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj] for src, obj in zip(SOURCES, objs)]
    if verbose:
        for cmd in cmds:
            print(" ".join(cmd), flush=True)
    # The sources compile independently: run the compiler processes side by side.
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        results = list(pool.map(lambda c: subprocess.run(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), cmds))
    for cmd, r in zip(cmds, results):
        if r.returncode != 0:
            sys.stderr.write(r.stdout.decode(errors="replace"))
            raise subprocess.CalledProcessError(r.returncode, cmd)
    tmp = LIB_PATH + ".tmp"
    # -z defs: every symbol the library uses must resolve at link time (a missing
    # launcher would otherwise surface only when the library is loaded).
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_host_sanitized(outdir: str, verbose: bool = False) -> str:
    """The library with its host code (argument checks, plans, launchers) compiled with AddressSanitizer and
    UndefinedBehaviorSanitizer, into outdir/libnvfp4_hostsan.so, for sweeping the C ABI's validation on a
    machine without a GPU.  The device code is built as usual (no sanitizer reaches it)."""
    cc = hipcc()
    os.makedirs(outdir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    flags = [*compile_flags(), *san]
    objs = [os.path.join(outdir, src + ".host.o") for src in SOURCES]
    cmds = [[cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj] for src, obj in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        results = list(pool.map(lambda c: subprocess.run(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), cmds))
    for cmd, r in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout.decode(errors="replace"))
            raise subprocess.CalledProcessError(r.returncode, cmd)
    lib = os.path.join(outdir, "libnvfp4_hostsan.so")
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
            "-fsanitize=undefined", "-o", lib, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
