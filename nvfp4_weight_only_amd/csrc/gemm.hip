// W4A16 prefill GEMM on bf16 MFMA, gfx950.
//
// The engine's prefill linear is a dense GEMM over the NVFP4 weights (imp
// "docs/quantization.md", NVFP4 kernel pipeline: prefill through an FP4
// tensor-core GEMM with a re-laid scale-factor layout).  gfx950 has no MFMA
// that takes E4M3 micro-scales per 16 elements, so weight tiles are
// dequantized into LDS as BF16 (E2M1 * E4M3 is exact in BF16) and multiplied
// with v_mfma_f32_16x16x32_bf16 in FP32; the tensor scale is applied in the
// epilogue.
//
// Tiling: a workgroup computes a BM x BN tile of Y = X W^T with WM x WN
// wavefronts; each wavefront owns (BM/WM) x (BN/WN) as 16x16 MFMA tiles.
// The K loop stages BK columns of X (BF16) and of W (dequantized) in LDS.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Prefill GEMM: 128 x 272 tiles, producer and consumer wavefronts.
//
// N = 17 * 1024 for the engine's MLP shapes, so a 272-wide tile (17 MFMA
// columns of 16) gives 64 tiles along N: 256 workgroups at M = 512 and 1024
// at M = 2048, i.e. whole waves of the 256 CUs.
//
// A workgroup has 8 wavefronts, two per SIMD:
//   consumers (0..3): 2 x 2 layout; wm picks 64 of the 128 rows, the column
//     half is MFMA columns 0..8 or 9..16.  They only read fragments from LDS
//     and issue v_mfma_f32_16x16x32_bf16;
//   producers (4..7): fetch the activations and packed weights of step kt + 2
//     into registers, dequantize step kt + 1 (exact BF16 E2M1 x E4M3) and
//     write it to the other LDS buffer.
// With one of each per SIMD, the MFMA pipe and the VALU work concurrently.
// BK = 64 columns of K per step; one barrier per step.
// ---------------------------------------------------------------------------
constexpr int kPfBM = 128, kPfBN = 272, kPfBK = 64, kPfLDK = kPfBK;  // LDS row: 128 bytes, no padding
constexpr int kPfThreads = 512, kPfProducers = 256;
constexpr int kPfXChunks = kPfBM * kPfBK / 8 / kPfProducers;                 // uint4 of X per producer thread (4)
constexpr int kPfWItems = kPfBN * (kPfBK / 16);                               // 16-element blocks per step (1088)
constexpr int kPfWPerThread = (kPfWItems + kPfProducers - 1) / kPfProducers;  // 5 (the 5th round: 64 items)
constexpr int kPfWRows = kPfBN;

// Producer work items: X chunk c -> (row c / 8, 16-byte column c % 8); weight
// item it -> (row it / 4, 16-element block it % 4), so every 64-lane load
// instruction reads whole 128-byte (X) or 32-byte (W) row segments.
__device__ __forceinline__ int pf_x_row(int c) { return c >> 3; }
__device__ __forceinline__ int pf_x_col8(int c) { return c & 7; }
__device__ __forceinline__ int pf_w_row(int it) { return it >> 2; }
__device__ __forceinline__ int pf_w_blk(int it) { return it & 3; }

// LDS layout: 16-byte chunk q of row r lives at chunk q ^ ((r >> 1) & 7) of
// the 128-byte row.  With 64 banks of 4 bytes this makes conflict-free both
// the MFMA fragment reads (16 consecutive rows, one chunk) and the producer
// writes (4 rows x 4 weight blocks, or 2 rows x 8 activation chunks, per 16 lanes).
__device__ __forceinline__ int pf_swz(int row, int q) { return row * kPfLDK + ((q ^ ((row >> 1) & 7)) << 3); }

struct PrefillArgs {
  const uint16_t* x;
  int64_t m, n, k;
  const uint8_t* packed;
  const uint8_t* scales;
  const float* tscale;
  uint16_t* y;
};

struct PrefillStage {
  uint4 xr[kPfXChunks];
  uint2 wr[kPfWPerThread];
  uint32_t sr[kPfWPerThread];
};

// Loads of step kt (out-of-range elements read a clamped in-bounds address and are then zeroed).
__device__ __forceinline__ void prefill_fetch(const PrefillArgs& p, int64_t m0, int64_t n0, int kt, int pt,
                                              PrefillStage& st) {
  const int64_t k0 = (int64_t)kt * kPfBK, kblocks = p.k >> 4, pstride = p.k >> 1;
#pragma unroll
  for (int i = 0; i < kPfXChunks; ++i) {
    const int c = pt + i * kPfProducers, row = pf_x_row(c), c8 = pf_x_col8(c);
    const int64_t gm = m0 + row, gk = k0 + c8 * 8;
    const bool ok = gm < p.m && gk < p.k;
    const int64_t cm = gm < p.m ? gm : p.m - 1, ck = gk < p.k ? gk : p.k - 8;
    const uint4 v = *reinterpret_cast<const uint4*>(p.x + cm * p.k + ck);
    st.xr[i] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < kPfWPerThread; ++i) {
    const int it = pt + i * kPfProducers, row = pf_w_row(it), b = pf_w_blk(it);
    if (it >= kPfWItems) break;  // uniform: only the first producer wavefront has a fifth item
    const int64_t gn = n0 + row, gb = (k0 >> 4) + b;
    const bool ok = gn < p.n && gb < kblocks;
    const int64_t cn = gn < p.n ? gn : p.n - 1, cb = gb < kblocks ? gb : kblocks - 1;
    const uint2 v = *reinterpret_cast<const uint2*>(p.packed + cn * pstride + cb * 8);
    const uint32_t sc = p.scales[cn * kblocks + cb];
    st.wr[i] = ok ? v : make_uint2(0u, 0u);
    st.sr[i] = ok ? sc : 0u;
  }
}

__device__ __forceinline__ void prefill_stash(uint16_t* xs, uint16_t* ws, int pt, const PrefillStage& st) {
#pragma unroll
  for (int i = 0; i < kPfXChunks; ++i) {
    const int c = pt + i * kPfProducers;
    *reinterpret_cast<uint4*>(&xs[pf_swz(pf_x_row(c), pf_x_col8(c))]) = st.xr[i];
  }
#pragma unroll
  for (int i = 0; i < kPfWPerThread; ++i) {
    const int it = pt + i * kPfProducers;
    if (it >= kPfWItems) break;  // uniform per wavefront
    const int row = pf_w_row(it), b = pf_w_blk(it);
    const float sc = e4m3x2_to_f32<false>(st.sr[i]).x;
    *reinterpret_cast<uint4*>(&ws[pf_swz(row, 2 * b)]) = e2m1x8_scaled_to_bf16_hw(st.wr[i].x, sc);
    *reinterpret_cast<uint4*>(&ws[pf_swz(row, 2 * b + 1)]) = e2m1x8_scaled_to_bf16_hw(st.wr[i].y, sc);
  }
}

typedef uint16_t PfXBuf[kPfBM * kPfLDK];
typedef uint16_t PfWBuf[kPfWRows * kPfLDK];

// Per-thread offsets of the producer's loads inside a tile; constant across K
// steps (the step only moves the uniform base pointers).
struct PrefillOffsets {
  uint32_t xo[kPfXChunks];     // elements, from x + m0 * k + k0
  uint32_t wo[kPfWPerThread];  // bytes, from packed + n0 * k/2 + k0/2
  uint32_t so[kPfWPerThread];  // bytes, from scales + n0 * k/16 + k0/16
};

// Loads of a step that lies fully inside the matrices: no per-element checks.
__device__ __forceinline__ void prefill_fetch_full(const PrefillArgs& p, int64_t m0, int64_t n0, int kt, int pt,
                                                   const PrefillOffsets& o, PrefillStage& st) {
  const int64_t k0 = (int64_t)kt * kPfBK;
  const uint16_t* xb = p.x + m0 * p.k + k0;
  const uint8_t* wb = p.packed + n0 * (p.k >> 1) + (k0 >> 1);
  const uint8_t* sb = p.scales + n0 * (p.k >> 4) + (k0 >> 4);
#pragma unroll
  for (int i = 0; i < kPfXChunks; ++i) st.xr[i] = *reinterpret_cast<const uint4*>(xb + o.xo[i]);
#pragma unroll
  for (int i = 0; i < kPfWPerThread; ++i) {
    if (pt + i * kPfProducers >= kPfWItems) break;  // uniform per wavefront
    st.wr[i] = *reinterpret_cast<const uint2*>(wb + o.wo[i]);
    st.sr[i] = sb[o.so[i]];
  }
}

__device__ __forceinline__ void prefill_producer(const PrefillArgs& p, PfXBuf* xs, PfWBuf* ws, int64_t m0,
                                                 int64_t n0, int ksteps) {
  const int pt = threadIdx.x - (kPfThreads - kPfProducers);
  const bool full_mn = m0 + kPfBM <= p.m && n0 + kPfBN <= p.n;
  PrefillOffsets o;
#pragma unroll
  for (int i = 0; i < kPfXChunks; ++i) {
    const int c = pt + i * kPfProducers;
    o.xo[i] = (uint32_t)(pf_x_row(c) * p.k + pf_x_col8(c) * 8);
  }
#pragma unroll
  for (int i = 0; i < kPfWPerThread; ++i) {
    const int it = pt + i * kPfProducers;
    o.wo[i] = (uint32_t)(pf_w_row(it) * (p.k >> 1) + pf_w_blk(it) * 8);
    o.so[i] = (uint32_t)(pf_w_row(it) * (p.k >> 4) + pf_w_blk(it));
  }
  // Steps past the end fetch nothing (their stash writes a buffer that is never read).
  auto fetch = [&](int kt, PrefillStage& st) {
    if (full_mn && (int64_t)(kt + 1) * kPfBK <= p.k)
      prefill_fetch_full(p, m0, n0, kt, pt, o, st);
    else if (kt < ksteps)
      prefill_fetch(p, m0, n0, kt, pt, st);
  };
  // Ring of four register stages: at step kt the producer fetches step kt + 4
  // into stage kt % 4 and dequantizes step kt + 1 (fetched three steps earlier)
  // into LDS buffer (kt + 1) & 1.
  PrefillStage st[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fetch(i, st[i]);
  prefill_stash(xs[0], ws[0], pt, st[0]);
  __syncthreads();
  for (int kt = 0; kt < ksteps; kt += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (kt + u < ksteps) {
        fetch(kt + u + 4, st[u]);
        prefill_stash(xs[(u + 1) & 1], ws[(u + 1) & 1], pt, st[(u + 1) & 3]);
        __syncthreads();
      }
    }
  }
}

template <int NC, int COL0>
__device__ __forceinline__ void prefill_consumer_step(const uint16_t* xb, const uint16_t* wb, int wm, int lane,
                                                      f32x4_t (&acc)[4][NC]) {
  constexpr int S = 2 * NC;
  // Row bases are multiples of 16, so the swizzle term depends on the lane only.
  const int swz = ((lane & 15) >> 1) & 7;
  const int c0 = ((lane >> 4) ^ swz) << 3, c1 = ((4 + (lane >> 4)) ^ swz) << 3;  // halves h = 0, 1
  const uint16_t* arow = xb + (wm * 64 + (lane & 15)) * kPfLDK;
  const uint16_t* brow = wb + (COL0 * 16 + (lane & 15)) * kPfLDK;
  auto ld = [](const uint16_t* q) { return *reinterpret_cast<const bf16x8_t*>(q); };
  constexpr int D = 4;  // prefetch distance in slots (ring of D + 1 B fragments)
  bf16x8_t a[2][4], b[D + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[0][i] = ld(arow + i * 16 * kPfLDK + c0);
#pragma unroll
  for (int d = 0; d < D; ++d) b[d] = ld(brow + (d % NC) * 16 * kPfLDK + (d / NC ? c1 : c0));
#pragma unroll
  for (int sidx = 0; sidx < S; ++sidx) {
    const int h = sidx / NC, j = sidx % NC;
    const int nx = sidx + D;
    if (nx < S) b[nx % (D + 1)] = ld(brow + (nx % NC) * 16 * kPfLDK + (nx / NC ? c1 : c0));
    if (sidx == NC - D) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[1][i] = ld(arow + i * 16 * kPfLDK + c1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[h][i], b[sidx % (D + 1)], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NC, int COL0>
__device__ __forceinline__ void prefill_consumer(const PrefillArgs& p, const PfXBuf* xs, const PfWBuf* ws,
                                                 int64_t m0, int64_t n0, int wm, int ksteps) {
  const int lane = threadIdx.x & 63;
  f32x4_t acc[4][NC];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    const int buf = kt & 1;
    prefill_consumer_step<NC, COL0>(xs[buf], ws[buf], wm, lane, acc);
    __syncthreads();
  }
  // D layout of a 16x16 MFMA tile: lane holds rows 4*(lane/16) + r, column lane % 16.
  const float t = *p.tscale;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int64_t gn = n0 + (COL0 + j) * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gm = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (gm < p.m && gn < p.n) p.y[gm * p.n + gn] = (uint16_t)f32_to_bf16_rne(acc[i][j][r] * t);
      }
  }
}

__global__ void __launch_bounds__(kPfThreads) prefill_kernel(PrefillArgs p) {
  __shared__ __attribute__((aligned(16))) PfXBuf xs[2];
  __shared__ __attribute__((aligned(16))) PfWBuf ws[2];
  const int wid = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * kPfBM, n0 = (int64_t)blockIdx.x * kPfBN;
  const int ksteps = (int)((p.k + kPfBK - 1) / kPfBK);
  // Every wavefront meets the same 1 + ksteps barriers.
  if (wid >= 4)
    prefill_producer(p, xs, ws, m0, n0, ksteps);
  else if (wid < 2)
    prefill_consumer<9, 0>(p, xs, ws, m0, n0, wid & 1, ksteps);
  else
    prefill_consumer<8, 9>(p, xs, ws, m0, n0, wid & 1, ksteps);
}

void launch_gemm_prefill(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                         const uint8_t* scales, const float* tscale, uint16_t* y, void* workspace,
                         int64_t workspace_bytes, hipStream_t s) {
  if (prefill_dma_supported(m, n, k))
    return launch_prefill_dma(x, m, n, k, packed, scales, tscale, y, workspace, workspace_bytes, s);
  const unsigned gx = (unsigned)((n + kPfBN - 1) / kPfBN);
  const int64_t tiles_m = (m + kPfBM - 1) / kPfBM;
  const int64_t max_y = 65535;
  for (int64_t t0 = 0; t0 < tiles_m; t0 += max_y) {
    const int64_t ty = (tiles_m - t0) < max_y ? (tiles_m - t0) : max_y;
    const int64_t mm = (m - t0 * kPfBM) < ty * kPfBM ? (m - t0 * kPfBM) : ty * kPfBM;
    const PrefillArgs p{x + t0 * kPfBM * k, mm, n, k, packed, scales, tscale, y + t0 * kPfBM * n};
    prefill_kernel<<<dim3(gx, (unsigned)ty), kPfThreads, 0, s>>>(p);
  }
}

}  // namespace nvfp4
