"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source's host part is compiled with both sanitizers (nvfp4_weight_only_amd.build.build_host_sanitized), and
tests/sanitize/abi_driver.cpp calls every entry point with null, misaligned and aliasing pointers and sizes from
-1 to INT64_MAX: any out-of-bounds access or undefined operation (signed overflow in a size computation, a bad
shift) aborts the driver.  The pointers are fake and never dereferenced, so the driver refuses to sweep when a GPU
is present (a call that passed validation would then launch)."""
import os
import shutil
import subprocess

import pytest

from nvfp4_weight_only_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rocm_clang():
    cc = B.hipcc()
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(cc)))
    path = os.path.join(rocm, "lib", "llvm", "bin", "clang++")
    return path if os.path.exists(path) else None, rocm


def test_abi_validation_under_asan_ubsan(tmp_path):
    clang, rocm = _rocm_clang()
    if clang is None:
        pytest.skip("ROCm clang++ not found")
    lib = B.build_host_sanitized(str(tmp_path))
    exe = str(tmp_path / "abi_driver")
    subprocess.run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), lib, "-o", exe,
                    "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"),
                    "-Wl,-rpath," + str(tmp_path)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "calls" in out or "skipped" in out, out[-2000:]
