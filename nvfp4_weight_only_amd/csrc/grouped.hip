// Grouped (routed) linear over an expert stack for many tokens: the prefill of
// a mixture-of-experts layer (imp "docs/quantization.md", NVFP4 kernel
// pipeline: a MoE layer's per-expert weights as one [ne, N, K_packed] buffer
// per layer and projection).  The (token, slot) pairs of the top-k routing are
// sorted by expert on the device; the prefill GEMM then runs over each
// expert's pairs in 128-row tiles, reading the activation row of each pair and
// writing its output row.
//
// Workspace (int32, caller-owned): cnt[E] (used only when E is too large for
// LDS), pair_off[E + 1], tile_off[E + 1], perm[pairs].  One workgroup sorts
// (counters, and for small problems the permutation, in LDS):
//   1. cnt[e] = number of pairs routed to e (ids outside [0, E) not counted);
//   2. pair_off / tile_off = exclusive prefix sums of cnt and ceil(cnt / 128);
//      pair_off[E] = V, the number of pairs with a valid id;
//   3. perm[pair_off[e] + cursor_e++] = pair for the valid pairs, and
//      perm[V + cursor_invalid++] = pair for the others.
// The grouped GEMM reads this: tiles of the valid pairs, and, in workgroups
// past the last tile, zeroes the output rows listed in perm[V .. pairs).
// The order of pairs inside an expert depends on the atomics; every output
// element is computed from its own activation row and weight row only, so
// the results do not.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {
namespace {

constexpr int kSortThreads = 1024, kSortWaves = kSortThreads / 64;
// LDS layouts of the sort: counters for up to 8192 experts; or counters for
// up to 1024 experts and the whole permutation for up to 32768 pairs (the
// scattered 4-byte stores then go to LDS, and perm leaves in coalesced rows).
constexpr int64_t kSortLdsExperts = 8192;
constexpr int64_t kSortPermExperts = 1024, kSortPermPairs = 32768;

// Counter access for the workspace form: loads and stores at device scope (past
// the vector L1, where the atomics act), and a device-scope fence before each
// barrier after which other wavefronts read them.
__device__ __forceinline__ int32_t ld_agent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The expert ids of pairs p0, p0 + 1024, ... (kSortBatch of them; -1 past the
// end), loaded together so that their latencies overlap.
constexpr int kSortBatch = 16;
__device__ __forceinline__ void sort_load_batch(const int32_t* __restrict__ route, int64_t pairs, int64_t p0,
                                                int32_t (&e)[kSortBatch]) {
#pragma unroll
  for (int i = 0; i < kSortBatch; ++i) {
    const int64_t p = p0 + (int64_t)i * kSortThreads;
    e[i] = p < pairs ? route[p] : -1;
  }
}

// CNT: capacity of the LDS counters (0: counters in the workspace); PERM:
// capacity of the LDS permutation (0: scattered straight to the workspace).
template <int CNT, int PERM>
__global__ void __launch_bounds__(kSortThreads) grp_sort_kernel(const int32_t* __restrict__ route, int64_t pairs,
                                                                int64_t experts, int32_t* ws) {
  constexpr bool LDS = CNT > 0;
  __shared__ int32_t lcnt[LDS ? CNT : 1];
  __shared__ int32_t lperm[PERM > 0 ? PERM : 1];
  __shared__ int32_t wsum[2][kSortWaves];
  __shared__ int32_t inv_cursor, valid_total;
  int32_t* cnt = LDS ? lcnt : ws;
  int32_t* pair_off = ws + experts;
  int32_t* tile_off = ws + 2 * experts + 1;
  int32_t* perm = ws + 3 * experts + 2;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  for (int64_t e = tid; e < experts; e += kSortThreads) {
    if constexpr (LDS) cnt[e] = 0;
    else st_agent(cnt + e, 0);
  }
  if (tid == 0) inv_cursor = 0;
  if constexpr (!LDS) __threadfence();
  __syncthreads();
  for (int64_t b = 0; b < pairs; b += kSortThreads * kSortBatch) {
    int32_t e[kSortBatch];
    sort_load_batch(route, pairs, b + tid, e);
#pragma unroll
    for (int i = 0; i < kSortBatch; ++i)
      if (e[i] >= 0 && (int64_t)e[i] < experts) atomicAdd(&cnt[e[i]], 1);
  }
  if constexpr (!LDS) __threadfence();
  __syncthreads();

  // Exclusive scan: thread tid owns experts [lo, hi); wavefront scans of the
  // per-thread sums, then the totals of the wavefronts before it.
  const int64_t per = (experts + kSortThreads - 1) / kSortThreads;
  const int64_t lo = tid * per < experts ? tid * per : experts;
  const int64_t hi = lo + per < experts ? lo + per : experts;
  int32_t sp = 0, st = 0;
  for (int64_t e = lo; e < hi; ++e) {
    const int32_t c = LDS ? cnt[e] : ld_agent(cnt + e);
    sp += c;
    st += (c + 127) >> 7;
  }
  int32_t ip = sp, it = st;  // inclusive within the wavefront
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t up = __shfl_up(ip, d, 64), ut = __shfl_up(it, d, 64);
    if (lane >= d) {
      ip += up;
      it += ut;
    }
  }
  if (lane == 63) {
    wsum[0][wv] = ip;
    wsum[1][wv] = it;
  }
  __syncthreads();
  int32_t bp = 0, bt = 0;
  for (int i = 0; i < wv; ++i) {
    bp += wsum[0][i];
    bt += wsum[1][i];
  }
  int32_t rp = bp + ip - sp, rt = bt + it - st;  // exclusive prefix of this thread's first expert
  for (int64_t e = lo; e < hi; ++e) {
    const int32_t c = LDS ? cnt[e] : ld_agent(cnt + e);
    pair_off[e] = rp;
    tile_off[e] = rt;
    if constexpr (LDS) cnt[e] = rp;  // from here on: the expert's cursor
    else st_agent(cnt + e, rp);
    rp += c;
    rt += (c + 127) >> 7;
  }
  if (tid == kSortThreads - 1) {
    pair_off[experts] = bp + ip;
    tile_off[experts] = bt + it;
    valid_total = bp + ip;
  }
  if constexpr (!LDS) __threadfence();
  __syncthreads();

  const int32_t v = valid_total;
  for (int64_t b = 0; b < pairs; b += kSortThreads * kSortBatch) {
    int32_t e[kSortBatch];
    sort_load_batch(route, pairs, b + tid, e);
#pragma unroll
    for (int i = 0; i < kSortBatch; ++i) {
      const int64_t p = b + tid + (int64_t)i * kSortThreads;
      if (p < pairs) {
        const bool ok = e[i] >= 0 && (int64_t)e[i] < experts;
        const int32_t pos = ok ? atomicAdd(&cnt[e[i]], 1) : v + atomicAdd(&inv_cursor, 1);
        if constexpr (PERM > 0) lperm[pos] = (int32_t)p;
        else perm[pos] = (int32_t)p;
      }
    }
  }
  if constexpr (PERM > 0) {
    __syncthreads();
    for (int64_t i = tid; i < pairs; i += kSortThreads) perm[i] = lperm[i];
  }
}

}  // namespace

int64_t grouped_workspace_bytes(int64_t pairs, int64_t experts) {
  return ((3 * experts + 2 + pairs) * 4 + 15) / 16 * 16;
}

void launch_linear_grouped(const uint16_t* x, int64_t t_count, int64_t topk, const int32_t* route, int64_t experts,
                           int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales, const float* tscale,
                           uint16_t* y, void* workspace, hipStream_t s) {
  const int64_t pairs = t_count * topk;
  int32_t* ws = static_cast<int32_t*>(workspace);
  if (experts <= kSortPermExperts && pairs <= kSortPermPairs)
    grp_sort_kernel<kSortPermExperts, kSortPermPairs><<<1, kSortThreads, 0, s>>>(route, pairs, experts, ws);
  else if (experts <= kSortLdsExperts)
    grp_sort_kernel<kSortLdsExperts, 0><<<1, kSortThreads, 0, s>>>(route, pairs, experts, ws);
  else
    grp_sort_kernel<0, 0><<<1, kSortThreads, 0, s>>>(route, pairs, experts, ws);
  launch_prefill_grouped(x, topk, ws, pairs, experts, n, k, packed, scales, tscale, y, s);
}

}  // namespace nvfp4
