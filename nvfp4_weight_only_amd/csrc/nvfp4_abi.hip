// C ABI of libnvfp4.so: argument validation, device check, kernel dispatch.
// Declarations and the meaning of every argument are in include/nvfp4.h.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "launch.hpp"
#include "nvfp4.h"

namespace {

constexpr int64_t kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges).
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

// a * b fits in int64 (a, b >= 0).
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

struct WeightSizes {
  int64_t elems, w_bytes, packed_bytes, scale_bytes;
};

nvfp4_status weight_sizes(int64_t n, int64_t k, WeightSizes* s) {
  if (n <= 0 || k <= 0 || (k & 15) != 0) return NVFP4_ERR_SHAPE;
  if (!mul_ok(n, k, &s->elems) || !mul_ok(s->elems, 2, &s->w_bytes)) return NVFP4_ERR_SHAPE;
  s->packed_bytes = s->elems / 2;
  s->scale_bytes = s->elems / 16;
  return NVFP4_OK;
}

// Checks that the current device is a gfx950 (cached per device).
nvfp4_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_DEVICE;
  int st = g_device_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NVFP4_ERR_DEVICE;
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? NVFP4_OK : NVFP4_ERR_UNSUPPORTED;
}

nvfp4_status launch_status() { return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE; }

nvfp4_status validate_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                             const uint8_t* scales, const float* tscale, const uint16_t* y) {
  // m = 0 is a no-op: x and y may then be NULL (empty tensors).
  if (!packed || !scales || !tscale || (m != 0 && (!x || !y))) return NVFP4_ERR_NULL;
  WeightSizes ws;
  if (m < 0) return NVFP4_ERR_SHAPE;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  if (m == 0) return NVFP4_OK;
  int64_t xe, ye, xb, yb;
  if (!mul_ok(m, k, &xe) || !mul_ok(xe, 2, &xb) || !mul_ok(m, n, &ye) || !mul_ok(ye, 2, &yb)) return NVFP4_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(scales) || !aligned16(tscale) || !aligned16(y))
    return NVFP4_ERR_ALIGN;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, packed, ws.packed_bytes) || overlaps(y, yb, scales, ws.scale_bytes) ||
      overlaps(y, yb, tscale, 4))
    return NVFP4_ERR_ALIAS;
  return NVFP4_OK;
}

int auto_kernel(int64_t m) {
  return m == 1 ? NVFP4_KERNEL_GEMV : (m <= 64 ? NVFP4_KERNEL_SMALL_M : NVFP4_KERNEL_PREFILL);
}

// A workspace is used by the small-M kernel and the prefill GEMM (K split across workgroups).
nvfp4_status run_linear(int kernel, const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                        const uint8_t* scales, const float* tscale, uint16_t* y, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  if (kernel < NVFP4_KERNEL_AUTO || kernel > NVFP4_KERNEL_PREFILL) return NVFP4_ERR_UNSUPPORTED;
  nvfp4_status st = validate_linear(x, m, n, k, packed, scales, tscale, y);
  if (st != NVFP4_OK) return st;
  if (workspace_bytes < 0) return NVFP4_ERR_SHAPE;
  if (workspace != nullptr && workspace_bytes > 0) {
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    int64_t xb = 0, yb = 0, pb = n * (k / 2), sb = n * (k / 16);
    mul_ok(m, 2 * k, &xb);
    mul_ok(m, 2 * n, &yb);
    if (overlaps(workspace, workspace_bytes, x, xb) || overlaps(workspace, workspace_bytes, y, yb) ||
        overlaps(workspace, workspace_bytes, packed, pb) || overlaps(workspace, workspace_bytes, scales, sb) ||
        overlaps(workspace, workspace_bytes, tscale, 4))
      return NVFP4_ERR_ALIAS;
  }
  if (m == 0) return NVFP4_OK;
  if ((st = check_device()) != NVFP4_OK) return st;
  if (kernel == NVFP4_KERNEL_AUTO) kernel = auto_kernel(m);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (kernel) {
    case NVFP4_KERNEL_GEMV: nvfp4::launch_gemv(x, m, n, k, packed, scales, tscale, y, s); break;
    case NVFP4_KERNEL_SMALL_M:
      nvfp4::launch_skinny(x, m, n, k, packed, scales, tscale, y, workspace, workspace ? workspace_bytes : 0, s);
      break;
    default:
      nvfp4::launch_gemm_prefill(x, m, n, k, packed, scales, tscale, y, workspace, workspace ? workspace_bytes : 0, s);
      break;
  }
  return launch_status();
}

nvfp4_status validate_quantize_outputs(const uint16_t* w, const WeightSizes& ws, const uint8_t* packed,
                                       const uint8_t* scales, const float* tscale) {
  if (!aligned16(w) || !aligned16(packed) || !aligned16(scales) || !aligned16(tscale)) return NVFP4_ERR_ALIGN;
  const void* outs[3] = {packed, scales, tscale};
  const int64_t out_bytes[3] = {ws.packed_bytes, ws.scale_bytes, 4};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], out_bytes[i], w, ws.w_bytes)) return NVFP4_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return NVFP4_ERR_ALIAS;
  }
  return NVFP4_OK;
}

// MXFP4 sizes of a rows x k tensor (k a multiple of 32; rows = 0 allowed).
nvfp4_status mx_sizes(int64_t rows, int64_t k, WeightSizes* s) {
  if (rows < 0 || k <= 0 || (k & 31) != 0) return NVFP4_ERR_SHAPE;
  if (!mul_ok(rows, k, &s->elems) || !mul_ok(s->elems, 2, &s->w_bytes)) return NVFP4_ERR_SHAPE;
  s->packed_bytes = s->elems / 2;
  s->scale_bytes = s->elems / 32;
  return NVFP4_OK;
}

int64_t mx_round16(int64_t b) { return (b + 15) / 16 * 16; }

// ---------------------------------------------------------------------------
// Library-owned scratch for nvfp4_linear_noalloc: the split-K workspace of the
// small-M kernel (arrival counters, then FP32 partial sums) in a file-scope
// device array, so that the call allocates nothing.  Every GPU the library
// runs on holds its own copy of the array until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: host code uses
// only the device address that hipGetSymbolAddress returns for the current
// device (kept per device below).
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = 8 << 20;   // covers every split the small-M kernel plans (at most 6.7 MiB)
__device__ __align__(256) uint8_t scratch[kScratchBytes];

void* g_scratch_ptr[kMaxDevices];
std::atomic<int> g_scratch_ready[kMaxDevices];  // 0 not set up, 1 set up
std::mutex g_scratch_mutex;

__global__ void zero_words_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The current device's copy of `scratch` (set up once per device: its address,
// and the arrival-counter region cleared by a kernel on `s`, which the caller's
// first call then follows in stream order).  NULL on a HIP error.
void* scratch_for_current_device(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (g_scratch_ready[dev].load(std::memory_order_acquire) == 1) return g_scratch_ptr[dev];
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ready[dev].load(std::memory_order_relaxed) == 1) return g_scratch_ptr[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
  zero_words_kernel<<<16, 256, 0, s>>>(static_cast<uint32_t*>(ptr), nvfp4::kSkinnyCounterBytes / 4);
  if (hipGetLastError() != hipSuccess) return nullptr;
  g_scratch_ptr[dev] = ptr;
  g_scratch_ready[dev].store(1, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL: a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE: invalid m/n/k (k must be a positive multiple of 16) or size overflow";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN: a pointer is not 16-byte aligned";
    case NVFP4_ERR_ALIAS: return "NVFP4_ERR_ALIAS: an output overlaps an input";
    case NVFP4_ERR_DEVICE: return "NVFP4_ERR_DEVICE: HIP error";
    case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED: device is not gfx950 or unknown kernel id";
    default: return "NVFP4_ERR_UNKNOWN";
  }
}

const char* nvfp4_version(void) { return "nvfp4-mi355x 0.1.0"; }

nvfp4_status nvfp4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* packed, uint8_t* scales, float* tscale,
                            void* stream) {
  if (!w || !packed || !scales || !tscale) return NVFP4_ERR_NULL;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  if ((st = validate_quantize_outputs(w, ws, packed, scales, tscale)) != NVFP4_OK) return st;
  if ((st = check_device()) != NVFP4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The packed output (n k / 2 bytes) holds the per-workgroup maxima until the
  // quantize pass overwrites it; the reduction writes the tensor scale, from
  // which the quantize pass recovers amax exactly.
  nvfp4::launch_tscale_set_stack(w, 1, ws.elems, reinterpret_cast<uint32_t*>(packed), tscale, s);
  nvfp4::launch_quantize_from_tscale(w, 1, ws.elems, tscale, packed, scales, s);
  return launch_status();
}

int64_t nvfp4_quantize_workspace_bytes(void) { return 4096; }

nvfp4_status nvfp4_quantize_ws(const uint16_t* w, int64_t n, int64_t k, uint8_t* packed, uint8_t* scales,
                               float* tscale, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!w || !packed || !scales || !tscale) return NVFP4_ERR_NULL;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  if ((st = validate_quantize_outputs(w, ws, packed, scales, tscale)) != NVFP4_OK) return st;
  if (workspace_bytes < 0) return NVFP4_ERR_SHAPE;
  if (workspace == nullptr || workspace_bytes < nvfp4_quantize_workspace_bytes())
    return nvfp4_quantize(w, n, k, packed, scales, tscale, stream);
  if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
  if (overlaps(workspace, workspace_bytes, w, ws.w_bytes) || overlaps(workspace, workspace_bytes, packed, ws.packed_bytes) ||
      overlaps(workspace, workspace_bytes, scales, ws.scale_bytes) || overlaps(workspace, workspace_bytes, tscale, 4))
    return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The per-workgroup maxima in the workspace: every encode workgroup reads them.
  nvfp4::launch_quantize_shared_amax(w, ws.elems, static_cast<uint32_t*>(workspace), tscale, packed, scales, s);
  return launch_status();
}

nvfp4_status nvfp4_amax_accumulate(const uint16_t* w, int64_t n, int64_t k, float* amax, void* stream) {
  if (!w || !amax) return NVFP4_ERR_NULL;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  if (!aligned16(w) || !aligned16(amax)) return NVFP4_ERR_ALIGN;
  if (overlaps(amax, 4, w, ws.w_bytes)) return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_amax(w, ws.elems, amax, static_cast<hipStream_t>(stream));
  return launch_status();
}

nvfp4_status nvfp4_quantize_with_amax(const uint16_t* w, int64_t n, int64_t k, const float* amax, uint8_t* packed,
                                      uint8_t* scales, float* tscale, void* stream) {
  if (!w || !amax || !packed || !scales || !tscale) return NVFP4_ERR_NULL;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  if (!aligned16(amax)) return NVFP4_ERR_ALIGN;
  if ((st = validate_quantize_outputs(w, ws, packed, scales, tscale)) != NVFP4_OK) return st;
  if (overlaps(amax, 4, packed, ws.packed_bytes) || overlaps(amax, 4, scales, ws.scale_bytes) ||
      overlaps(amax, 4, tscale, 4))
    return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  nvfp4::launch_quantize(w, 1, ws.elems, amax, packed, scales, s);
  nvfp4::launch_finalize_tscale(amax, tscale, 1, s);
  return launch_status();
}

nvfp4_status nvfp4_dequant(const uint8_t* packed, const uint8_t* scales, const float* tscale, int64_t n, int64_t k,
                           uint16_t* w_out, void* stream) {
  if (!packed || !scales || !tscale || !w_out) return NVFP4_ERR_NULL;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  if (!aligned16(packed) || !aligned16(scales) || !aligned16(tscale) || !aligned16(w_out)) return NVFP4_ERR_ALIGN;
  if (overlaps(w_out, ws.w_bytes, packed, ws.packed_bytes) || overlaps(w_out, ws.w_bytes, scales, ws.scale_bytes) ||
      overlaps(w_out, ws.w_bytes, tscale, 4))
    return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_dequant(packed, scales, tscale, 1, ws.elems, w_out, static_cast<hipStream_t>(stream));
  return launch_status();
}

nvfp4_status nvfp4_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                          const uint8_t* scales, const float* tscale, uint16_t* y, void* stream) {
  return run_linear(NVFP4_KERNEL_AUTO, x, m, n, k, packed, scales, tscale, y, nullptr, 0, stream);
}

int64_t nvfp4_linear_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  WeightSizes ws;
  if (m < 0 || weight_sizes(n, k, &ws) != NVFP4_OK) return -1;
  int64_t ye;
  if (!mul_ok(m, n, &ye) || ye > INT64_MAX / 32) return -1;
  const int kernel = auto_kernel(m);
  if (kernel == NVFP4_KERNEL_PREFILL) return nvfp4::prefill_workspace_bytes(m, n, k);
  if (kernel != NVFP4_KERNEL_SMALL_M) return 0;
  return nvfp4::skinny_workspace_bytes(m, n, k);
}

nvfp4_status nvfp4_linear_ws(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                             const uint8_t* scales, const float* tscale, uint16_t* y, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  return run_linear(NVFP4_KERNEL_AUTO, x, m, n, k, packed, scales, tscale, y, workspace, workspace_bytes, stream);
}

int64_t nvfp4_linear_noalloc_max_bytes(void) { return kScratchBytes; }

nvfp4_status nvfp4_linear_noalloc(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                                  const uint8_t* scales, const float* tscale, uint16_t* y, void* stream) {
  nvfp4_status st = validate_linear(x, m, n, k, packed, scales, tscale, y);
  if (st != NVFP4_OK) return st;
  if (m == 0) return NVFP4_OK;
  // The scratch array serves the small-M kernel's K split; the prefill GEMM
  // runs unsplit here (its split needs more than the array holds).
  const int64_t need = auto_kernel(m) == NVFP4_KERNEL_PREFILL ? 0 : nvfp4_linear_workspace_bytes(m, n, k);
  if (need < 0 || need > kScratchBytes) return NVFP4_ERR_SHAPE;
  if ((st = check_device()) != NVFP4_OK) return st;
  if (need == 0) return run_linear(NVFP4_KERNEL_AUTO, x, m, n, k, packed, scales, tscale, y, nullptr, 0, stream);
  void* ws = scratch_for_current_device(static_cast<hipStream_t>(stream));
  if (ws == nullptr) return NVFP4_ERR_DEVICE;
  return run_linear(NVFP4_KERNEL_AUTO, x, m, n, k, packed, scales, tscale, y, ws, kScratchBytes, stream);
}

int64_t nvfp4_prepared_bytes(int64_t n, int64_t k) {
  WeightSizes ws;
  if (weight_sizes(n, k, &ws) != NVFP4_OK || k % 128 != 0) return -1;
  const int64_t tiles = (n + 15) / 16;
  int64_t b;
  if (!mul_ok(tiles, k / 128, &b) || !mul_ok(b, 1152, &b)) return -1;
  return b;
}

nvfp4_status nvfp4_prepare(const uint8_t* packed, const uint8_t* scales, int64_t n, int64_t k, uint8_t* prepared,
                           void* stream) {
  if (!packed || !scales || !prepared) return NVFP4_ERR_NULL;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  const int64_t pb = nvfp4_prepared_bytes(n, k);
  if (pb < 0) return NVFP4_ERR_SHAPE;
  if (!aligned16(packed) || !aligned16(scales) || !aligned16(prepared)) return NVFP4_ERR_ALIGN;
  if (overlaps(prepared, pb, packed, ws.packed_bytes) || overlaps(prepared, pb, scales, ws.scale_bytes))
    return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_prepare(packed, scales, n, k, prepared, static_cast<hipStream_t>(stream));
  return launch_status();
}

nvfp4_status nvfp4_dequant_prepared(const uint8_t* prepared, const float* tscale, int64_t n, int64_t k,
                                    uint16_t* w_out, void* stream) {
  if (!prepared || !tscale || !w_out) return NVFP4_ERR_NULL;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  const int64_t pb = nvfp4_prepared_bytes(n, k);
  if (pb < 0) return NVFP4_ERR_SHAPE;
  if (!aligned16(prepared) || !aligned16(tscale) || !aligned16(w_out)) return NVFP4_ERR_ALIGN;
  if (overlaps(w_out, ws.w_bytes, prepared, pb) || overlaps(w_out, ws.w_bytes, tscale, 4)) return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_dequant_prepared(prepared, tscale, n, k, w_out, static_cast<hipStream_t>(stream));
  return launch_status();
}

int64_t nvfp4_linear_prepared_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || nvfp4_prepared_bytes(n, k) < 0) return -1;
  int64_t ye;
  if (!mul_ok(m, n, &ye) || ye > INT64_MAX / 32) return -1;
  if (m <= 1 || !nvfp4::small_m_supported(m, n, k)) return 0;  // m = 1: the prepared GEMV takes none
  return nvfp4::small_m_plan(m, n, k, true).ws_bytes;
}

nvfp4_status nvfp4_linear_prepared(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* prepared,
                                   const float* tscale, uint16_t* y, void* workspace, int64_t workspace_bytes,
                                   void* stream) {
  if (!prepared || !tscale || (m != 0 && (!x || !y))) return NVFP4_ERR_NULL;
  if (m < 0 || workspace_bytes < 0) return NVFP4_ERR_SHAPE;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  const int64_t pb = nvfp4_prepared_bytes(n, k);
  if (pb < 0) return NVFP4_ERR_SHAPE;
  int64_t xe, ye, xb, yb;
  if (!mul_ok(m, k, &xe) || !mul_ok(xe, 2, &xb) || !mul_ok(m, n, &ye) || !mul_ok(ye, 2, &yb)) return NVFP4_ERR_SHAPE;
  if (m == 0) return NVFP4_OK;
  if (!nvfp4::small_m_supported(m, n, k)) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(prepared) || !aligned16(tscale) || !aligned16(y)) return NVFP4_ERR_ALIGN;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, prepared, pb) || overlaps(y, yb, tscale, 4)) return NVFP4_ERR_ALIAS;
  if (m == 1) {
    if ((st = check_device()) != NVFP4_OK) return st;
    nvfp4::launch_gemv_prepared(x, n, k, prepared, tscale, y, static_cast<hipStream_t>(stream));
    return launch_status();
  }
  nvfp4::SmallMPlan pl = nvfp4::small_m_plan(m, n, k, true);
  if (pl.slices > 1 && (workspace == nullptr || workspace_bytes < pl.ws_bytes)) pl = nvfp4::small_m_plan(m, n, k, false);
  if (pl.slices > 1) {
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    if (overlaps(workspace, workspace_bytes, x, xb) || overlaps(workspace, workspace_bytes, y, yb) ||
        overlaps(workspace, workspace_bytes, prepared, pb) || overlaps(workspace, workspace_bytes, tscale, 4))
      return NVFP4_ERR_ALIAS;
  }
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_small_m(pl, x, m, n, k, prepared, tscale, y, workspace, static_cast<hipStream_t>(stream));
  return launch_status();
}

int64_t nvfp4_stream_read_sink_words(int64_t bytes) {
  if (bytes <= 0 || bytes % 16 != 0) return -1;
  return nvfp4::stream_read_blocks(bytes);
}

nvfp4_status nvfp4_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return NVFP4_ERR_NULL;
  if (bytes <= 0 || bytes % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return NVFP4_ERR_ALIGN;
  if (overlaps(sink, 4 * nvfp4::stream_read_blocks(bytes), src, bytes)) return NVFP4_ERR_ALIAS;
  nvfp4_status st;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream));
  return launch_status();
}

nvfp4_status nvfp4_linear_forced(int kernel_id, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                 const uint8_t* packed, const uint8_t* scales, const float* tscale, uint16_t* y,
                                 void* stream) {
  return run_linear(kernel_id, x, m, n, k, packed, scales, tscale, y, nullptr, 0, stream);
}

nvfp4_status nvfp4_quantize_experts(const uint16_t* w, int64_t e, int64_t n, int64_t k, uint8_t* packed,
                                    uint8_t* scales, float* tscale, void* stream) {
  if (!w || !packed || !scales || !tscale) return NVFP4_ERR_NULL;
  if (e < 0 || e > 65535) return NVFP4_ERR_SHAPE;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  WeightSizes all;  // the whole stack
  if (!mul_ok(ws.elems, e, &all.elems) || !mul_ok(all.elems, 2, &all.w_bytes)) return NVFP4_ERR_SHAPE;
  all.packed_bytes = all.elems / 2;
  all.scale_bytes = all.elems / 16;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(scales) || !aligned16(tscale)) return NVFP4_ERR_ALIGN;
  const void* outs[3] = {packed, scales, tscale};
  const int64_t out_bytes[3] = {all.packed_bytes, all.scale_bytes, 4 * e};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], out_bytes[i], w, all.w_bytes)) return NVFP4_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return NVFP4_ERR_ALIAS;
  }
  if (e == 0) return NVFP4_OK;
  if ((st = check_device()) != NVFP4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  nvfp4::launch_tscale_set_stack(w, e, ws.elems, reinterpret_cast<uint32_t*>(packed), tscale, s);
  nvfp4::launch_quantize_from_tscale(w, e, ws.elems, tscale, packed, scales, s);
  return launch_status();
}

nvfp4_status nvfp4_dequant_experts(const uint8_t* packed, const uint8_t* scales, const float* tscale, int64_t e,
                                   int64_t n, int64_t k, uint16_t* w_out, void* stream) {
  if (!packed || !scales || !tscale || !w_out) return NVFP4_ERR_NULL;
  if (e < 0 || e > 65535) return NVFP4_ERR_SHAPE;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  int64_t elems, w_bytes;
  if (!mul_ok(ws.elems, e, &elems) || !mul_ok(elems, 2, &w_bytes)) return NVFP4_ERR_SHAPE;
  if (!aligned16(packed) || !aligned16(scales) || !aligned16(tscale) || !aligned16(w_out)) return NVFP4_ERR_ALIGN;
  if (overlaps(w_out, w_bytes, packed, elems / 2) || overlaps(w_out, w_bytes, scales, elems / 16) ||
      overlaps(w_out, w_bytes, tscale, 4 * e))
    return NVFP4_ERR_ALIAS;
  if (e == 0) return NVFP4_OK;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_dequant(packed, scales, tscale, e, ws.elems, w_out, static_cast<hipStream_t>(stream));
  return launch_status();
}

nvfp4_status nvfp4_linear_routed(const uint16_t* x, int64_t t_count, int64_t topk, const int32_t* route, int64_t e,
                                 int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                                 const float* tscale, uint16_t* y, void* stream) {
  if (!packed || !scales || !tscale || (t_count != 0 && (!x || !route || !y))) return NVFP4_ERR_NULL;
  if (t_count < 0 || topk < 1 || e < 1) return NVFP4_ERR_SHAPE;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  int64_t elems, pairs, xe, xb, ye, yb;
  if (!mul_ok(ws.elems, e, &elems) || !mul_ok(t_count, topk, &pairs) || !mul_ok(t_count, k, &xe) ||
      !mul_ok(xe, 2, &xb) || !mul_ok(pairs, n, &ye) || !mul_ok(ye, 2, &yb) || pairs > INT64_MAX / 4)
    return NVFP4_ERR_SHAPE;
  if (t_count == 0) return NVFP4_OK;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(scales) || !aligned16(tscale) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(route) & 3u) != 0)
    return NVFP4_ERR_ALIGN;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, route, 4 * pairs) || overlaps(y, yb, packed, elems / 2) ||
      overlaps(y, yb, scales, elems / 16) || overlaps(y, yb, tscale, 4 * e))
    return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_gemv_routed(x, t_count, topk, route, e, n, k, packed, scales, tscale, y,
                            static_cast<hipStream_t>(stream));
  return launch_status();
}

int64_t nvfp4_linear_grouped_workspace_bytes(int64_t t_count, int64_t topk, int64_t e) {
  int64_t pairs;
  if (t_count < 0 || topk < 1 || e < 1 || !mul_ok(t_count, topk, &pairs) || pairs > INT64_MAX / 8 ||
      e > INT64_MAX / 32)
    return -1;
  return nvfp4::grouped_workspace_bytes(pairs, e);
}

nvfp4_status nvfp4_linear_grouped(const uint16_t* x, int64_t t_count, int64_t topk, const int32_t* route, int64_t e,
                                  int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                                  const float* tscale, uint16_t* y, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
  if (!packed || !scales || !tscale || (t_count != 0 && (!x || !route || !y || !workspace))) return NVFP4_ERR_NULL;
  if (t_count < 0 || topk < 1 || e < 1) return NVFP4_ERR_SHAPE;
  WeightSizes ws;
  nvfp4_status st = weight_sizes(n, k, &ws);
  if (st != NVFP4_OK) return st;
  int64_t elems, pairs, xe, xb, ye, yb;
  if (!mul_ok(ws.elems, e, &elems) || !mul_ok(t_count, topk, &pairs) || !mul_ok(t_count, k, &xe) ||
      !mul_ok(xe, 2, &xb) || !mul_ok(pairs, n, &ye) || !mul_ok(ye, 2, &yb) || pairs > INT64_MAX / 8 ||
      e > INT64_MAX / 32)
    return NVFP4_ERR_SHAPE;
  const int64_t need = nvfp4::grouped_workspace_bytes(pairs, e);
  if (t_count == 0) return NVFP4_OK;
  if (workspace_bytes < need) return NVFP4_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(scales) || !aligned16(tscale) || !aligned16(y) ||
      !aligned16(workspace) || (reinterpret_cast<uintptr_t>(route) & 3u) != 0)
    return NVFP4_ERR_ALIGN;
  const void* ins[5] = {x, route, packed, scales, tscale};
  const int64_t in_bytes[5] = {xb, 4 * pairs, elems / 2, elems / 16, 4 * e};
  for (int i = 0; i < 5; ++i)
    if (overlaps(y, yb, ins[i], in_bytes[i]) || overlaps(workspace, need, ins[i], in_bytes[i]))
      return NVFP4_ERR_ALIAS;
  if (overlaps(workspace, need, y, yb)) return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nvfp4::prefill_grouped_supported(t_count, topk, e, n, k))
    nvfp4::launch_linear_grouped(x, t_count, topk, route, e, n, k, packed, scales, tscale, y, workspace, s);
  else
    nvfp4::launch_gemv_routed(x, t_count, topk, route, e, n, k, packed, scales, tscale, y, s);
  return launch_status();
}

nvfp4_status nvfp4_kv_gather(int format, int out_type, const uint8_t* codes, const uint8_t* scales,
                             const float* tscale, int64_t num_blocks, int64_t block_size, int64_t heads,
                             int64_t head_dim, const int32_t* block_table, int64_t max_blocks,
                             const int32_t* seq_lens, const int32_t* dst_start, int64_t seqs, uint16_t* out,
                             int64_t out_rows, void* stream) {
  if ((format != NVFP4_KV_NVFP4 && format != NVFP4_KV_MXFP4) || (out_type != NVFP4_OUT_F16 && out_type != NVFP4_OUT_BF16))
    return NVFP4_ERR_UNSUPPORTED;
  const bool mx = format == NVFP4_KV_MXFP4;
  if (!codes || !scales || (!mx && !tscale) || (seqs != 0 && (!block_table || !seq_lens || !dst_start || !out)))
    return NVFP4_ERR_NULL;
  const int64_t group = mx ? 32 : 16;
  if (num_blocks < 1 || block_size < 1 || heads < 1 || head_dim < 1 || head_dim % group != 0 || max_blocks < 1 ||
      seqs < 0 || out_rows < 0)
    return NVFP4_ERR_SHAPE;
  int64_t row_elems, page_elems, cache_elems, tab, ob;
  if (!mul_ok(heads, head_dim, &row_elems) || !mul_ok(row_elems, block_size, &page_elems) ||
      !mul_ok(page_elems, num_blocks, &cache_elems) || !mul_ok(seqs, max_blocks, &tab) || tab > INT32_MAX ||
      tab > INT64_MAX / 4 || !mul_ok(out_rows, row_elems, &ob) || ob > INT64_MAX / 2 ||
      max_blocks > INT64_MAX / block_size)
    return NVFP4_ERR_SHAPE;
  ob *= 2;
  if (seqs == 0) return NVFP4_OK;
  if (!aligned16(codes) || !aligned16(out) || (reinterpret_cast<uintptr_t>(tscale) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(dst_start) & 3u) != 0)
    return NVFP4_ERR_ALIGN;
  if (overlaps(out, ob, codes, cache_elems / 2) || overlaps(out, ob, scales, cache_elems / group) ||
      (!mx && overlaps(out, ob, tscale, 4)) || overlaps(out, ob, block_table, 4 * tab) ||
      overlaps(out, ob, seq_lens, 4 * seqs) || overlaps(out, ob, dst_start, 4 * seqs))
    return NVFP4_ERR_ALIAS;
  nvfp4_status st;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_kv_gather(mx, out_type == NVFP4_OUT_BF16, codes, scales, tscale, num_blocks, block_size, row_elems,
                          block_table, max_blocks, seq_lens, dst_start, seqs, out, out_rows,
                          static_cast<hipStream_t>(stream));
  return launch_status();
}

nvfp4_status nvfp4_mx_quantize(const uint16_t* w, int64_t rows, int64_t k, uint8_t* packed, uint8_t* scales,
                               void* stream) {
  WeightSizes ws;
  nvfp4_status st = mx_sizes(rows, k, &ws);
  if (st != NVFP4_OK) return st;
  if (rows == 0) return NVFP4_OK;
  if (!w || !packed || !scales) return NVFP4_ERR_NULL;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(scales)) return NVFP4_ERR_ALIGN;
  if (overlaps(packed, ws.packed_bytes, w, ws.w_bytes) || overlaps(scales, ws.scale_bytes, w, ws.w_bytes) ||
      overlaps(packed, ws.packed_bytes, scales, ws.scale_bytes))
    return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_mx_quantize(w, rows, k, packed, scales, static_cast<hipStream_t>(stream));
  return launch_status();
}

nvfp4_status nvfp4_mx_dequant(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, uint16_t* out,
                              void* stream) {
  WeightSizes ws;
  nvfp4_status st = mx_sizes(rows, k, &ws);
  if (st != NVFP4_OK) return st;
  if (rows == 0) return NVFP4_OK;
  if (!packed || !scales || !out) return NVFP4_ERR_NULL;
  if (!aligned16(packed) || !aligned16(scales) || !aligned16(out)) return NVFP4_ERR_ALIGN;
  if (overlaps(out, ws.w_bytes, packed, ws.packed_bytes) || overlaps(out, ws.w_bytes, scales, ws.scale_bytes))
    return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_mx_dequant(packed, scales, rows, k, out, static_cast<hipStream_t>(stream));
  return launch_status();
}

nvfp4_status nvfp4_mx_gemm(const uint8_t* xq, const uint8_t* xs, int64_t m, const uint8_t* wq, const uint8_t* ws,
                           int64_t n, int64_t k, uint16_t* y, void* stream) {
  WeightSizes xsz, wsz;
  nvfp4_status st;
  if ((st = mx_sizes(m, k, &xsz)) != NVFP4_OK || (st = mx_sizes(n, k, &wsz)) != NVFP4_OK) return st;
  if (n == 0) return NVFP4_ERR_SHAPE;
  int64_t ye, yb;
  if (!mul_ok(m, n, &ye) || !mul_ok(ye, 2, &yb)) return NVFP4_ERR_SHAPE;
  if (m == 0) return NVFP4_OK;
  if (!xq || !xs || !wq || !ws || !y) return NVFP4_ERR_NULL;
  if (!nvfp4::mx_gemm_supported(m, n, k)) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || !aligned16(y)) return NVFP4_ERR_ALIGN;
  if (overlaps(y, yb, xq, xsz.packed_bytes) || overlaps(y, yb, xs, xsz.scale_bytes) ||
      overlaps(y, yb, wq, wsz.packed_bytes) || overlaps(y, yb, ws, wsz.scale_bytes))
    return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  nvfp4::launch_mx_gemm(xq, xs, m, wq, ws, n, k, y, static_cast<hipStream_t>(stream));
  return launch_status();
}

int64_t nvfp4_mx_linear_w4a4_workspace_bytes(int64_t m, int64_t k) {
  WeightSizes xs;
  if (mx_sizes(m, k, &xs) != NVFP4_OK || xs.packed_bytes > INT64_MAX / 4) return -1;
  return mx_round16(xs.packed_bytes) + mx_round16(xs.scale_bytes);
}

nvfp4_status nvfp4_mx_linear_w4a4(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* wq,
                                  const uint8_t* ws, uint16_t* y, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
  WeightSizes xsz, wsz;
  nvfp4_status st;
  if ((st = mx_sizes(m, k, &xsz)) != NVFP4_OK || (st = mx_sizes(n, k, &wsz)) != NVFP4_OK) return st;
  if (n == 0 || workspace_bytes < 0) return NVFP4_ERR_SHAPE;
  int64_t ye, yb;
  if (!mul_ok(m, n, &ye) || !mul_ok(ye, 2, &yb) || xsz.packed_bytes > INT64_MAX / 4) return NVFP4_ERR_SHAPE;
  if (m == 0) return NVFP4_OK;
  if (!x || !wq || !ws || !y || !workspace) return NVFP4_ERR_NULL;
  const int64_t need = mx_round16(xsz.packed_bytes) + mx_round16(xsz.scale_bytes);
  if (workspace_bytes < need) return NVFP4_ERR_SHAPE;
  if (!nvfp4::mx_gemm_supported(m, n, k)) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(ws) || !aligned16(y) || !aligned16(workspace))
    return NVFP4_ERR_ALIGN;
  const void* ins[3] = {x, wq, ws};
  const int64_t in_bytes[3] = {xsz.w_bytes, wsz.packed_bytes, wsz.scale_bytes};
  for (int i = 0; i < 3; ++i)
    if (overlaps(y, yb, ins[i], in_bytes[i]) || overlaps(workspace, need, ins[i], in_bytes[i])) return NVFP4_ERR_ALIAS;
  if (overlaps(workspace, need, y, yb)) return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  uint8_t* xs = xq + mx_round16(xsz.packed_bytes);
  nvfp4::launch_mx_quantize(x, m, k, xq, xs, s);
  nvfp4::launch_mx_gemm(xq, xs, m, wq, ws, n, k, y, s);
  return launch_status();
}

// NVFP4 x NVFP4: workspace = X codes [m, k/2] | X scales [m, k/16] | {ts_y, amax_x, ts_x, -} | X decoded BF16 [m, k],
// each part starting on a 16-byte boundary.
int64_t nvfp4_linear_w4a4_workspace_bytes(int64_t m, int64_t k) {
  WeightSizes xs;
  if (m < 0 || k <= 0 || (k & 15) != 0) return -1;
  if (m == 0) return 0;
  if (weight_sizes(m, k, &xs) != NVFP4_OK || xs.w_bytes > INT64_MAX / 2) return -1;
  return mx_round16(xs.packed_bytes) + mx_round16(xs.scale_bytes) + 16 + xs.w_bytes;
}

nvfp4_status nvfp4_linear_w4a4(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                               const uint8_t* scales, const float* tscale, uint16_t* y, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  nvfp4_status st = validate_linear(x, m, n, k, packed, scales, tscale, y);
  if (st != NVFP4_OK) return st;
  if (workspace_bytes < 0) return NVFP4_ERR_SHAPE;
  if (m == 0) return NVFP4_OK;
  const int64_t need = nvfp4_linear_w4a4_workspace_bytes(m, k);
  if (need < 0) return NVFP4_ERR_SHAPE;
  if (!workspace) return NVFP4_ERR_NULL;
  if (workspace_bytes < need) return NVFP4_ERR_SHAPE;
  if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
  WeightSizes xs, wsz;
  weight_sizes(m, k, &xs);
  weight_sizes(n, k, &wsz);
  const void* bufs[5] = {x, y, packed, scales, tscale};
  const int64_t bytes[5] = {xs.w_bytes, 2 * m * n, wsz.packed_bytes, wsz.scale_bytes, 4};
  for (int i = 0; i < 5; ++i)
    if (overlaps(workspace, need, bufs[i], bytes[i])) return NVFP4_ERR_ALIAS;
  if ((st = check_device()) != NVFP4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  uint8_t* xsc = xq + mx_round16(xs.packed_bytes);
  float* f = reinterpret_cast<float*>(xsc + mx_round16(xs.scale_bytes));
  uint16_t* xd = reinterpret_cast<uint16_t*>(f + 4);
  // amax_x (per-workgroup maxima in the code buffer first), then codes + scales + decoded X and the two tensor
  // scales in one kernel, then the weight-only linear on the decoded X with ts_w * ts_x as its tensor scale.
  // ts_y sits first so that it is 16-byte aligned like every tensor scale the linear takes.
  nvfp4::launch_amax_set(x, xs.elems, reinterpret_cast<uint32_t*>(xq), f + 1, s);
  nvfp4::launch_quantize_decode(x, xs.elems, f + 1, xq, xsc, xd, tscale, f + 2, f, s);
  if (hipGetLastError() != hipSuccess) return NVFP4_ERR_DEVICE;
  return run_linear(NVFP4_KERNEL_AUTO, xd, m, n, k, packed, scales, f, y, nullptr, 0, stream);
}

}  // extern "C"
