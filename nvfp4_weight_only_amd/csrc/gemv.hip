// W4A16 GEMV for decode (M = 1; larger M runs row by row) on gfx950.
//
// The engine's decode linear is a bandwidth-bound GEMV over packed NVFP4
// weights (imp "docs/quantization.md", NVFP4 kernel pipeline: a GEMV with a
// byte-permute register lookup table, split along K).  Here:
//   - each wavefront owns RPW weight rows and streams them with 16-byte loads
//     (32 elements = two 16-element blocks per lane per row);
//   - the activation row is staged once per workgroup in LDS, pre-permuted so
//     that v_perm_b32 decodes of the packed nibbles pair up with it directly;
//   - nibbles are decoded with v_perm_b32 lookups into unscaled BF16 E2M1
//     values and multiplied with v_dot2_f32_bf16 (FP32 accumulate); the E4M3
//     block scale is applied once per 16 elements with an FMA, the tensor
//     scale once per output in the epilogue;
//   - the per-lane partial sums are reduced across the wavefront with shuffles.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int64_t kGemvChunk = 16384;  // K elements of the activation row staged in LDS at a time (32 KiB)

// UB = 16-element blocks per lane unit: 2 (16-byte loads, needs k % 32 == 0) or 1 (8-byte loads).
template <int RPW, int UB>
__global__ void __launch_bounds__(kGemvThreads) gemv_kernel(const uint16_t* __restrict__ x, int64_t n, int64_t k,
                                                            const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ tscale_p,
                                                            uint16_t* __restrict__ y) {
  __shared__ uint4 xs[kGemvChunk / 8];  // permuted activations, 8 per uint4
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t mrow = blockIdx.y;
  const uint16_t* xr = x + mrow * k;
  const int64_t row0 = ((int64_t)blockIdx.x * kGemvWaves + wid) * RPW;
  const int64_t kblocks = k >> 4;
  const int64_t pstride = k >> 1;

  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;

  for (int64_t k0 = 0; k0 < k; k0 += kGemvChunk) {
    const int64_t kc = (k - k0) < kGemvChunk ? (k - k0) : kGemvChunk;  // multiple of 16
    __syncthreads();
    for (int64_t g = threadIdx.x; g < (kc >> 3); g += kGemvThreads)
      xs[g] = bf16x8_interleave(*reinterpret_cast<const uint4*>(xr + k0 + 8 * g));
    __syncthreads();

    const int64_t units = kc / (16 * UB);
    for (int64_t u = lane; u < units; u += 64) {
      uint4 xq[2 * UB];
#pragma unroll
      for (int q = 0; q < 2 * UB; ++q) xq[q] = xs[u * 2 * UB + q];
      const int64_t blk = (k0 >> 4) + u * UB;  // first block of the unit within the row
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int64_t row = row0 + r;
        if (row < n) {
          const uint8_t* prow = packed + row * pstride + blk * 8;
          const uint8_t* srow = scales + row * kblocks + blk;
          if constexpr (UB == 2) {
            const uint4 pk = *reinterpret_cast<const uint4*>(prow);
            const uint32_t sc = *reinterpret_cast<const uint16_t*>(srow);
            float p0 = 0.0f, p1 = 0.0f;
            uint4 d;
            d = e2m1x8_to_bf16_interleaved(pk.x);
            p0 = dot2_bf16(d.x, xq[0].x, p0); p0 = dot2_bf16(d.y, xq[0].y, p0);
            p0 = dot2_bf16(d.z, xq[0].z, p0); p0 = dot2_bf16(d.w, xq[0].w, p0);
            d = e2m1x8_to_bf16_interleaved(pk.y);
            p0 = dot2_bf16(d.x, xq[1].x, p0); p0 = dot2_bf16(d.y, xq[1].y, p0);
            p0 = dot2_bf16(d.z, xq[1].z, p0); p0 = dot2_bf16(d.w, xq[1].w, p0);
            d = e2m1x8_to_bf16_interleaved(pk.z);
            p1 = dot2_bf16(d.x, xq[2].x, p1); p1 = dot2_bf16(d.y, xq[2].y, p1);
            p1 = dot2_bf16(d.z, xq[2].z, p1); p1 = dot2_bf16(d.w, xq[2].w, p1);
            d = e2m1x8_to_bf16_interleaved(pk.w);
            p1 = dot2_bf16(d.x, xq[3].x, p1); p1 = dot2_bf16(d.y, xq[3].y, p1);
            p1 = dot2_bf16(d.z, xq[3].z, p1); p1 = dot2_bf16(d.w, xq[3].w, p1);
            acc[r] = fmaf(p0, e4m3_to_f32(sc & 0xFFu), acc[r]);
            acc[r] = fmaf(p1, e4m3_to_f32(sc >> 8), acc[r]);
          } else {
            const uint2 pk = *reinterpret_cast<const uint2*>(prow);
            const uint32_t sc = *srow;
            float p0 = 0.0f;
            uint4 d;
            d = e2m1x8_to_bf16_interleaved(pk.x);
            p0 = dot2_bf16(d.x, xq[0].x, p0); p0 = dot2_bf16(d.y, xq[0].y, p0);
            p0 = dot2_bf16(d.z, xq[0].z, p0); p0 = dot2_bf16(d.w, xq[0].w, p0);
            d = e2m1x8_to_bf16_interleaved(pk.y);
            p0 = dot2_bf16(d.x, xq[1].x, p0); p0 = dot2_bf16(d.y, xq[1].y, p0);
            p0 = dot2_bf16(d.z, xq[1].z, p0); p0 = dot2_bf16(d.w, xq[1].w, p0);
            acc[r] = fmaf(p0, e4m3_to_f32(sc), acc[r]);
          }
        }
      }
    }
  }

  const float t = *tscale_p;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float v = wave_sum(acc[r]);
    const int64_t row = row0 + r;
    if (lane == 0 && row < n) y[mrow * n + row] = (uint16_t)f32_to_bf16_rne(v * t);
  }
}

void launch_gemv(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                 const float* tscale, uint16_t* y, hipStream_t s) {
  constexpr int RPW = 4;
  const unsigned gx = (unsigned)((n + kGemvWaves * RPW - 1) / (kGemvWaves * RPW));
  const int64_t max_y = 65535;  // gridDim.y limit: activation rows go in slices
  for (int64_t m0 = 0; m0 < m; m0 += max_y) {
    const unsigned gy = (unsigned)((m - m0) < max_y ? (m - m0) : max_y);
    if ((k & 31) == 0)
      gemv_kernel<RPW, 2><<<dim3(gx, gy), kGemvThreads, 0, s>>>(x + m0 * k, n, k, packed, scales, tscale, y + m0 * n);
    else
      gemv_kernel<RPW, 1><<<dim3(gx, gy), kGemvThreads, 0, s>>>(x + m0 * k, n, k, packed, scales, tscale, y + m0 * n);
  }
}

}  // namespace nvfp4
