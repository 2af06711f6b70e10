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
  launch_tiles<128, 128, 64, 2, 2>(x, m, n, k, packed, scales, tscale, y, s);
}

}  // namespace nvfp4
