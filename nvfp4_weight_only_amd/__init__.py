"""MI355X-native NVFP4 weight-only (W4A16) linear.

The hot path runs in hand-written gfx950 HIP kernels behind the C ABI of
libnvfp4.so (include/nvfp4.h).  This package holds the kernels (csrc/), the
build script, the ctypes binding and the synthetic workload generators.
"""
from .binding import (KERNEL_IDS, KV_FORMATS, NVFP4Error, amax_accumulate, dequant, dequant_experts, kv_gather, lib,
                      lib_path, linear, linear_noalloc, linear_prepared, prepare, dequant_prepared, prepared_bytes, linear_w4a4, linear_w4a4_workspace_bytes, mx_dequant, mx_gemm, mx_linear_w4a4, mx_quantize,
                      linear_grouped, linear_grouped_workspace_bytes, linear_routed, linear_workspace_bytes,
                      quantize, quantize_experts, quantize_shared, quantize_with_amax)

__all__ = ["KERNEL_IDS", "KV_FORMATS", "NVFP4Error", "amax_accumulate", "dequant", "dequant_experts", "kv_gather",
           "lib", "lib_path", "linear", "linear_noalloc", "linear_prepared", "prepare", "dequant_prepared", "prepared_bytes", "linear_w4a4", "linear_w4a4_workspace_bytes", "mx_dequant", "mx_gemm", "mx_linear_w4a4", "mx_quantize",
           "linear_grouped", "linear_grouped_workspace_bytes", "linear_routed", "linear_workspace_bytes", "quantize", "quantize_experts", "quantize_shared",
           "quantize_with_amax"]
