// Grouped (routed) linear over an expert stack for many tokens: the prefill of
// a mixture-of-experts layer (imp "docs/quantization.md", NVFP4 kernel
// pipeline: a MoE layer's per-expert weights as one [ne, N, K_packed] buffer
// per layer and projection).  The (token, slot) pairs of the top-k routing are
// sorted by expert on the device; the prefill GEMM then runs over each
// expert's pairs in 128-row tiles, reading the activation row of each pair and
// writing its output row.
//
// Workspace (int32, caller-owned): counts[E], cursors[E], pair_off[E + 1],
// tile_off[E + 1], perm[pairs].  Kernels, in stream order:
//   1. grp_zero: counts and cursors = 0 (a fill kernel, so the sequence can be
//      captured in a graph);
//   2. grp_count: counts[e] = number of pairs routed to e (ids outside [0, E)
//      are not counted);
//   3. grp_scan: pair_off / tile_off = exclusive prefix sums of counts and of
//      ceil(counts / 128);
//   4. grp_scatter: perm[pair_off[e] + cursors[e]++] = pair; a pair with an
//      id outside [0, E) gets its output row zeroed instead;
//   5. the grouped prefill GEMM.
// The order of pairs inside an expert depends on the atomics, but every output
// element is computed from its own activation row and weight row only, so the
// results do not.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {
namespace {

constexpr int kGrpThreads = 256;

__global__ void __launch_bounds__(kGrpThreads) grp_zero_kernel(int32_t* a, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    a[i] = 0;
}

__global__ void __launch_bounds__(kGrpThreads) grp_count_kernel(const int32_t* __restrict__ route, int64_t pairs,
                                                                int64_t experts, int32_t* counts) {
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < pairs; p += (int64_t)gridDim.x * blockDim.x) {
    const int32_t e = route[p];
    if (e >= 0 && (int64_t)e < experts) atomicAdd(&counts[e], 1);
  }
}

// One workgroup; thread 0 walks the experts (E is small next to the GEMM).
__global__ void __launch_bounds__(64) grp_scan_kernel(const int32_t* __restrict__ counts, int64_t experts,
                                                      int32_t* pair_off, int32_t* tile_off) {
  if (threadIdx.x != 0) return;
  int32_t po = 0, to = 0;
  for (int64_t e = 0; e < experts; ++e) {
    pair_off[e] = po;
    tile_off[e] = to;
    const int32_t c = counts[e];
    po += c;
    to += (c + 127) / 128;
  }
  pair_off[experts] = po;
  tile_off[experts] = to;
}

__global__ void __launch_bounds__(kGrpThreads) grp_scatter_kernel(const int32_t* __restrict__ route, int64_t pairs,
                                                                  int64_t experts, const int32_t* __restrict__ pair_off,
                                                                  int32_t* cursors, int32_t* perm, uint16_t* y,
                                                                  int64_t n) {
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < pairs; p += (int64_t)gridDim.x * blockDim.x) {
    const int32_t e = route[p];
    if (e >= 0 && (int64_t)e < experts) {
      perm[pair_off[e] + atomicAdd(&cursors[e], 1)] = (int32_t)p;
    } else {
      for (int64_t j = 0; j < n; ++j) y[p * n + j] = 0;
    }
  }
}

unsigned grp_blocks(int64_t items) {
  const int64_t b = (items + kGrpThreads - 1) / kGrpThreads;
  return (unsigned)(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

}  // namespace

int64_t grouped_workspace_bytes(int64_t pairs, int64_t experts) {
  return ((4 * experts + 2 + pairs) * 4 + 15) / 16 * 16;
}

void launch_linear_grouped(const uint16_t* x, int64_t t_count, int64_t topk, const int32_t* route, int64_t experts,
                           int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales, const float* tscale,
                           uint16_t* y, void* workspace, hipStream_t s) {
  const int64_t pairs = t_count * topk;
  int32_t* ints = static_cast<int32_t*>(workspace);
  int32_t* counts = ints;
  int32_t* cursors = ints + experts;
  int32_t* pair_off = ints + 2 * experts;
  int32_t* tile_off = ints + 3 * experts + 1;
  int32_t* perm = ints + 4 * experts + 2;
  grp_zero_kernel<<<grp_blocks(2 * experts), kGrpThreads, 0, s>>>(counts, 2 * experts);
  grp_count_kernel<<<grp_blocks(pairs), kGrpThreads, 0, s>>>(route, pairs, experts, counts);
  grp_scan_kernel<<<1, 64, 0, s>>>(counts, experts, pair_off, tile_off);
  grp_scatter_kernel<<<grp_blocks(pairs), kGrpThreads, 0, s>>>(route, pairs, experts, pair_off, cursors, perm, y, n);
  (void)tile_off;
  launch_prefill_grouped(x, topk, ints, pairs, experts, n, k, packed, scales, tscale, y, s);
}

}  // namespace nvfp4
