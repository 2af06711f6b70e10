"""MI355X-native NVFP4 weight-only (W4A16) linear: HIP kernels behind a C ABI, with a thin binding."""
