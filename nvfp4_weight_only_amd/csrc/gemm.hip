// W4A16 GEMM on bf16 MFMA for batched decode (small M) and prefill (large M), gfx950.
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

template <int BM, int BN, int BK, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) gemm_kernel(const uint16_t* __restrict__ x, int64_t m, int64_t n,
                                                            int64_t k, const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ tscale_p,
                                                            uint16_t* __restrict__ y) {
  constexpr int NT = 64 * WM * WN;
  constexpr int LDK = BK + 8;  // padded LDS row (elements); 16-byte aligned rows
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  static_assert(TM >= 1 && TN >= 1 && BK % 32 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t xs[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t ws[BN * LDK];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t kblocks = k >> 4;
  const int64_t pstride = k >> 1;

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int64_t k0 = 0; k0 < k; k0 += BK) {
    __syncthreads();
    // X tile: BM rows x BK columns in 8-element chunks (zero outside [m, k)).
    for (int c = threadIdx.x; c < BM * (BK / 8); c += NT) {
      const int r = c / (BK / 8), cc = c % (BK / 8);
      const int64_t gm = m0 + r, gk = k0 + cc * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (gm < m && gk < k) v = *reinterpret_cast<const uint4*>(x + gm * k + gk);
      *reinterpret_cast<uint4*>(xs + r * LDK + cc * 8) = v;
    }
    // W tile: BN rows x BK columns, one 16-element block (8 packed bytes + 1 scale) per item.
    for (int c = threadIdx.x; c < BN * (BK / 16); c += NT) {
      const int r = c / (BK / 16), bb = c % (BK / 16);
      const int64_t gn = n0 + r, gb = (k0 >> 4) + bb;
      uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
      if (gn < n && gb < kblocks) {
        const uint2 pk = *reinterpret_cast<const uint2*>(packed + gn * pstride + gb * 8);
        const float s = e4m3_to_f32(scales[gn * kblocks + gb]);
        lo = e2m1x8_scaled_to_bf16(pk.x, s);
        hi = e2m1x8_scaled_to_bf16(pk.y, s);
      }
      *reinterpret_cast<uint4*>(ws + r * LDK + bb * 16) = lo;
      *reinterpret_cast<uint4*>(ws + r * LDK + bb * 16 + 8) = hi;
    }
    __syncthreads();

#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t a[TM], b[TN];
      const int koff = kk + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(xs + ((wm * TM + i) * 16 + (lane & 15)) * LDK + koff);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(ws + ((wn * TN + j) * 16 + (lane & 15)) * LDK + koff);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // D layout of a 16x16 MFMA tile: lane holds rows 4*(lane/16) + r, column lane % 16.
  const float t = *tscale_p;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gm = m0 + (wm * TM + i) * 16 + 4 * (lane >> 4) + r;
        const int64_t gn = n0 + (wn * TN + j) * 16 + (lane & 15);
        if (gm < m && gn < n) y[gm * n + gn] = (uint16_t)f32_to_bf16_rne(acc[i][j][r] * t);
      }
}

// ---------------------------------------------------------------------------
// Prefill GEMM: 128 x 272 tiles.  N = 17 * 1024 for the engine's MLP shapes,
// so a 272-wide tile (17 MFMA columns of 16) gives 64 tiles along N: 256
// workgroups at M = 512 and 1024 at M = 2048, i.e. whole waves of the 256 CUs.
// Four wavefronts in a 2 x 2 layout: wm picks 64 of the 128 rows, wn picks
// MFMA columns 0..8 or 9..16 of the tile.  BK = 64 columns of K per step,
// double-buffered in LDS; the next step's activations and packed weights are
// fetched into registers while the MFMAs of the current step run, then the
// weights are dequantized once per workgroup (exact BF16 E2M1 x E4M3) and
// written to the other buffer.
// ---------------------------------------------------------------------------
constexpr int kPfBM = 128, kPfBN = 272, kPfBK = 64, kPfLDK = kPfBK + 8;
constexpr int kPfThreads = 256;
constexpr int kPfXChunks = kPfBM * kPfBK / 8 / kPfThreads;              // uint4 of X per thread per step (4)
constexpr int kPfWItems = kPfBN * (kPfBK / 16);                          // 16-element blocks per step (1088)
constexpr int kPfWPerThread = (kPfWItems + kPfThreads - 1) / kPfThreads;  // 5

struct PrefillArgs {
  const uint16_t* x;
  int64_t m, n, k;
  const uint8_t* packed;
  const uint8_t* scales;
  const float* tscale;
  uint16_t* y;
};

// Staging of one K step: activations (BF16) and packed weights + scales.
struct PrefillStage {
  uint4 xr[kPfXChunks];
  uint2 wr[kPfWPerThread];
  uint32_t sr[kPfWPerThread];
};

__device__ __forceinline__ void prefill_fetch(const PrefillArgs& p, int64_t m0, int64_t n0, int kt, int tid,
                                              PrefillStage& st) {
  const int64_t k0 = (int64_t)kt * kPfBK, kblocks = p.k >> 4, pstride = p.k >> 1;
#pragma unroll
  for (int i = 0; i < kPfXChunks; ++i) {
    const int c = tid + i * kPfThreads, row = c >> 3, c8 = c & 7;
    const int64_t gm = m0 + row, gk = k0 + c8 * 8;
    st.xr[i] = (gm < p.m && gk < p.k) ? *reinterpret_cast<const uint4*>(p.x + gm * p.k + gk)
                                      : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < kPfWPerThread; ++i) {
    const int it = tid + i * kPfThreads, row = it >> 2, b = it & 3;
    const int64_t gn = n0 + row, gb = (k0 >> 4) + b;
    const bool ok = it < kPfWItems && gn < p.n && gb < kblocks;
    st.wr[i] = ok ? *reinterpret_cast<const uint2*>(p.packed + gn * pstride + gb * 8) : make_uint2(0u, 0u);
    st.sr[i] = ok ? p.scales[gn * kblocks + gb] : 0u;
  }
}

__device__ __forceinline__ void prefill_stash(uint16_t* xs, uint16_t* ws, int tid, const PrefillStage& st) {
#pragma unroll
  for (int i = 0; i < kPfXChunks; ++i) {
    const int c = tid + i * kPfThreads, row = c >> 3, c8 = c & 7;
    *reinterpret_cast<uint4*>(&xs[row * kPfLDK + c8 * 8]) = st.xr[i];
  }
#pragma unroll
  for (int i = 0; i < kPfWPerThread; ++i) {
    const int it = tid + i * kPfThreads, row = it >> 2, b = it & 3;
    if (it < kPfWItems) {
      const float sc = e4m3x2_to_f32<false>(st.sr[i]).x;
      *reinterpret_cast<uint4*>(&ws[row * kPfLDK + b * 16]) = e2m1x8_scaled_to_bf16_hw(st.wr[i].x, sc);
      *reinterpret_cast<uint4*>(&ws[row * kPfLDK + b * 16 + 8]) = e2m1x8_scaled_to_bf16_hw(st.wr[i].y, sc);
    }
  }
}

// Main loop and epilogue of one wavefront owning NC MFMA columns starting at COL0.
template <int NC, int COL0>
__device__ __forceinline__ void prefill_wave(const PrefillArgs& p, uint16_t (*xs)[kPfBM * kPfLDK],
                                             uint16_t (*ws)[kPfBN * kPfLDK], int64_t m0, int64_t n0, int wm) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int ksteps = (int)((p.k + kPfBK - 1) / kPfBK);
  f32x4_t acc[4][NC];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  PrefillStage st;
  prefill_fetch(p, m0, n0, 0, tid, st);
  prefill_stash(xs[0], ws[0], tid, st);
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < ksteps;
    if (more) prefill_fetch(p, m0, n0, kt + 1, tid, st);
#pragma unroll
    for (int kk = 0; kk < kPfBK; kk += 32) {
      const int koff = kk + 8 * (lane >> 4);
      bf16x8_t a[4], b[NC];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(&xs[buf][(wm * 64 + i * 16 + (lane & 15)) * kPfLDK + koff]);
#pragma unroll
      for (int j = 0; j < NC; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(&ws[buf][((COL0 + j) * 16 + (lane & 15)) * kPfLDK + koff]);
#pragma unroll
      for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) prefill_stash(xs[buf ^ 1], ws[buf ^ 1], tid, st);
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
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kPfBM * kPfLDK];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kPfBN * kPfLDK];
  const int wid = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * kPfBM, n0 = (int64_t)blockIdx.x * kPfBN;
  // wavefronts 0, 1: columns 0..8; wavefronts 2, 3: columns 9..16 (wid & 1 picks the 64-row half)
  if (wid < 2)
    prefill_wave<9, 0>(p, xs, ws, m0, n0, wid & 1);
  else
    prefill_wave<8, 9>(p, xs, ws, m0, n0, wid & 1);
}

template <int BM, int BN, int BK, int WM, int WN>
static void launch_tiles(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                         const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
  const unsigned gx = (unsigned)((n + BN - 1) / BN);
  const int64_t tiles_m = (m + BM - 1) / BM;
  // gridDim.y is limited; split very tall problems into several launches.
  const int64_t max_y = 65535;
  for (int64_t t0 = 0; t0 < tiles_m; t0 += max_y) {
    const int64_t ty = (tiles_m - t0) < max_y ? (tiles_m - t0) : max_y;
    const int64_t mm = (m - t0 * BM) < ty * BM ? (m - t0 * BM) : ty * BM;
    gemm_kernel<BM, BN, BK, WM, WN><<<dim3(gx, (unsigned)ty), 64 * WM * WN, 0, s>>>(
        x + t0 * BM * k, mm, n, k, packed, scales, tscale, y + t0 * BM * n);
  }
}

void launch_gemm_small_m(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                         const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
  if (m <= 16)
    launch_tiles<16, 64, 128, 1, 4>(x, m, n, k, packed, scales, tscale, y, s);
  else
    launch_tiles<32, 64, 128, 1, 4>(x, m, n, k, packed, scales, tscale, y, s);
}

void launch_gemm_prefill(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                         const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
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
