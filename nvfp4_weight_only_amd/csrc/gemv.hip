// W4A16 GEMV for decode (M = 1; larger M runs row by row) on gfx950.
//
// The engine's decode linear is a bandwidth-bound GEMV over packed NVFP4
// weights (imp "docs/quantization.md", NVFP4 kernel pipeline: a GEMV with a
// register lookup table, split along K).  Design for CDNA4:
//   - every lane issues all of its weight and scale loads (16-byte units of
//     32 elements = two 16-element blocks) before computing, so a whole launch
//     keeps the weights in flight;
//   - nibbles become BF16 pairs with one v_cvt_scalef32_pk_bf16_fp4 per byte
//     (scale 1.0: exact E2M1 values), products accumulate with
//     v_dot2_f32_bf16 in FP32; the E4M3 block scale is one FMA per 16
//     elements and the tensor scale one multiply per output.
// Four kernels, by k:
//   - gemv_ks_kernel (k a multiple of 512, k <= 5120): K split across the
//     wavefronts of a 12- or 16-row workgroup, one 512-element slice each,
//     activations and scales staged per wavefront with one wide load each, no
//     barrier before the products;
//   - gemv_ksl_kernel (k a multiple of 512, 5120 < k <= 32768): the same with
//     up to four slices per wavefront, all their loads issued first;
//   - gemv_lds_kernel (other k, a multiple of 32, up to 8192): each wavefront
//     owns whole rows, the activation row is staged once per workgroup in LDS;
//   - gemv_loop_kernel (any k a multiple of 16): rows per wavefront, K in
//     batches, activations read straight into registers.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;

// Routing over an expert stack (the MoE decode path): launch row blockIdx.y is
// pair p = pair0 + blockIdx.y; it reads activation row p / topk, writes output
// row p, and uses matrix route[p] of the stack (w_stride packed bytes,
// w_stride / 8 scale bytes, one tensor scale per matrix apart).  A pair whose
// expert id is outside [0, experts) writes zeros.
struct GvRoute {
  const int32_t* route;
  int64_t topk, experts, pair0, w_stride;
};

// One launch row resolved: activation row, output row and the matrix to use;
// ok is false when the pair's expert id is out of range.
struct GvRow {
  const uint16_t* x;
  uint16_t* y;
  const uint8_t* packed;
  const uint8_t* scales;
  const float* tscale;
  bool ok;
};

template <bool ROUTED>
__device__ __forceinline__ GvRow gv_resolve(const GvRoute& rt, const uint16_t* x, uint16_t* y, int64_t k, int64_t n,
                                            const uint8_t* packed, const uint8_t* scales, const float* tscale) {
  if constexpr (ROUTED) {
    const int64_t pair = rt.pair0 + blockIdx.y;
    const int32_t e = rt.route[pair];
    const bool ok = e >= 0 && (int64_t)e < rt.experts;
    const int64_t ee = ok ? e : 0;
    return GvRow{x + (pair / rt.topk) * k, y + pair * n, packed + ee * rt.w_stride, scales + ee * (rt.w_stride >> 3),
                 tscale + ee, ok};
  } else {
    return GvRow{x + (int64_t)blockIdx.y * k, y + (int64_t)blockIdx.y * n, packed, scales, tscale, true};
  }
}

// Dot product of one packed word (8 elements, natural order) with 8 activations.
__device__ __forceinline__ float dot8(uint32_t w, uint4 xq, float acc) {
  acc = dot2_bf16(e2m1x2_to_bf16<0>(w), xq.x, acc);
  acc = dot2_bf16(e2m1x2_to_bf16<1>(w), xq.y, acc);
  acc = dot2_bf16(e2m1x2_to_bf16<2>(w), xq.z, acc);
  acc = dot2_bf16(e2m1x2_to_bf16<3>(w), xq.w, acc);
  return acc;
}

// R rows per wavefront; JB units per lane per batch; UB = 16-element blocks per
// unit: 2 (16-byte loads, k % 32 == 0) or 1 (8-byte loads).
template <int R, int JB, int UB, bool ROUTED = false>
__global__ void __launch_bounds__(kGemvThreads) gemv_loop_kernel(const uint16_t* __restrict__ x, int64_t n, int64_t k,
                                                            const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ tscale_p,
                                                            uint16_t* __restrict__ y, GvRoute rt = GvRoute{}) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * kGemvWaves + (threadIdx.x >> 6)) * R;
  if (row0 >= n) return;  // uniform per wavefront
  {
    const GvRow rr = gv_resolve<ROUTED>(rt, x, y, k, n, packed, scales, tscale_p);
    y = rr.y;
    if (!rr.ok) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == 0 && row0 + r < n) y[row0 + r] = 0;
      return;
    }
    x = rr.x;
    packed = rr.packed;
    scales = rr.scales;
    tscale_p = rr.tscale;
  }
  const uint16_t* xr = x;
  const int64_t units = k / (16 * UB);
  const int64_t kblocks = k >> 4, pstride = k >> 1;

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  for (int64_t u0 = 0; u0 < units; u0 += 64 * JB) {
    uint32_t wv[JB][R][2 * UB];
    uint32_t sv[JB][R];
    uint4 xv[JB][2 * UB];
    // Weights and scales first: they come from HBM.
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int64_t u = u0 + 64 * j + lane;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r;
        if (u < units && row < n) {
          const uint8_t* pp = packed + row * pstride + u * 8 * UB;
          const uint8_t* sp = scales + row * kblocks + u * UB;
          if constexpr (UB == 2) {
            const uint4 v = *reinterpret_cast<const uint4*>(pp);
            wv[j][r][0] = v.x; wv[j][r][1] = v.y; wv[j][r][2] = v.z; wv[j][r][3] = v.w;
            sv[j][r] = *reinterpret_cast<const uint16_t*>(sp);
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(pp);
            wv[j][r][0] = v.x; wv[j][r][1] = v.y;
            sv[j][r] = *sp;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 2 * UB; ++q) wv[j][r][q] = 0u;
          sv[j][r] = 0u;
        }
      }
    }
    // Activations (shared by every wavefront: L2/L1 resident).
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int64_t u = u0 + 64 * j + lane;
#pragma unroll
      for (int q = 0; q < 2 * UB; ++q)
        xv[j][q] = (u < units) ? *reinterpret_cast<const uint4*>(xr + u * 16 * UB + 8 * q) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < UB; ++b) {
          float p = dot8(wv[j][r][2 * b], xv[j][2 * b], 0.0f);
          p = dot8(wv[j][r][2 * b + 1], xv[j][2 * b + 1], p);
          acc[r] = fmaf(p, e4m3_to_f32((sv[j][r] >> (8 * b)) & 0xFFu), acc[r]);
        }
  }

  const float t = *tscale_p;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = wave_sum(acc[r]);
    const int64_t row = row0 + r;
    if (lane == 0 && row < n) y[row] = (uint16_t)f32_to_bf16_rne(v * t);
  }
}

template <int R, int JB>
static void launch_rj(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                      const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
  const unsigned gx = (unsigned)((n + kGemvWaves * R - 1) / (kGemvWaves * R));
  const int64_t max_y = 65535;  // gridDim.y limit: activation rows go in slices
  for (int64_t m0 = 0; m0 < m; m0 += max_y) {
    const unsigned gy = (unsigned)((m - m0) < max_y ? (m - m0) : max_y);
    if ((k & 31) == 0)
      gemv_loop_kernel<R, JB, 2><<<dim3(gx, gy), kGemvThreads, 0, s>>>(x + m0 * k, n, k, packed, scales, tscale, y + m0 * n);
    else
      gemv_loop_kernel<R, JB, 1><<<dim3(gx, gy), kGemvThreads, 0, s>>>(x + m0 * k, n, k, packed, scales, tscale, y + m0 * n);
  }
}

// GEMV with the activation row staged in LDS (k % 32 == 0, k <= kLdsMaxK).
// Reading a small activation vector from every wavefront through the vector
// memory path makes a few L2 lines the hottest spot of the chip, so each
// workgroup of W wavefronts stages it once: every thread issues its share of
// activation loads, then all of its weight and scale loads, then writes the
// activations to LDS and meets the barrier (which waits only for LDS writes:
// the weight loads stay in flight).  Units are then consumed in issue order.
// LDS holds the activations quad-major (quad q of unit u at q * units + u), so
// lanes reading consecutive units touch consecutive banks.
constexpr int64_t kLdsMaxK = 16384;

template <int LPR, int R, int JB, int W, bool RAGGED>
__global__ void __launch_bounds__(64 * W) gemv_lds_kernel(const uint16_t* __restrict__ x, int64_t n, int64_t k,
                                                          const uint8_t* __restrict__ packed,
                                                          const uint8_t* __restrict__ scales,
                                                          const float* __restrict__ tscale_p,
                                                          uint16_t* __restrict__ y) {
  constexpr int SUB = 64 / LPR;
  constexpr int RPW = R * SUB;
  constexpr int NT = 64 * W;
  __shared__ uint4 xs[kLdsMaxK / 8];
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, ul = lane % LPR;
  const int units = (int)(k >> 5);
  const int64_t wrow0 = ((int64_t)blockIdx.x * W + (threadIdx.x >> 6)) * RPW;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)blockIdx.y * k);
  auto has = [&](int j) { return !RAGGED || ul + j * LPR < units; };

  // 1. activation loads (this thread's share of the k/8 uint4 of the row)
  constexpr int XPT = kLdsMaxK / 8 / NT + 1;  // upper bound of uint4 per thread
  uint4 xl[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int g = threadIdx.x + i * NT;
    xl[i] = g < (int)(k >> 3) ? xr[g] : make_uint4(0u, 0u, 0u, 0u);
  }
  // 2. weight and scale loads
  uint4 wv[JB][R];
  uint32_t sv[JB][R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = wrow0 + r * SUB + sub;
    const bool ok = row < n;
    const uint8_t* pb = packed + row * (k >> 1) + ul * 16;
    const uint8_t* sb = scales + row * (k >> 4) + ul * 2;
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const bool okj = ok && has(j);
      wv[j][r] = okj ? *reinterpret_cast<const uint4*>(pb + j * LPR * 16) : make_uint4(0u, 0u, 0u, 0u);
      sv[j][r] = okj ? *reinterpret_cast<const uint16_t*>(sb + j * LPR * 2) : 0u;
    }
  }
  // 3. activations to LDS, quad-major
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int g = threadIdx.x + i * NT;
    if (g < (int)(k >> 3)) xs[(g & 3) * units + (g >> 2)] = xl[i];
  }
  __syncthreads();
  if (wrow0 >= n) return;  // after the barrier: uniform per wavefront

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    if (!has(j)) continue;
    const int u = ul + j * LPR;
    const uint4 x0 = xs[u], x1 = xs[units + u], x2 = xs[2 * units + u], x3 = xs[3 * units + u];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float2 s = e4m3x2_to_f32<false>(sv[j][r]);
      float p0 = dot8(wv[j][r].x, x0, 0.0f);
      p0 = dot8(wv[j][r].y, x1, p0);
      float p1 = dot8(wv[j][r].z, x2, 0.0f);
      p1 = dot8(wv[j][r].w, x3, p1);
      acc[r] = fmaf(p0, s.x, acc[r]);
      acc[r] = fmaf(p1, s.y, acc[r]);
    }
  }

  const float t = *tscale_p;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = group_sum<LPR>(acc[r]);
    const int64_t row = wrow0 + r * SUB + sub;
    if (ul == 0 && row < n) y[(int64_t)blockIdx.y * n + row] = (uint16_t)f32_to_bf16_rne(v * t);
  }
}

// K-split GEMV (k % 512 == 0).  A workgroup owns 4 I consecutive rows and
// splits K across its W wavefronts: wavefront w owns the slice of 16 J units
// (a unit is 32 elements: 16 packed bytes, 2 scale bytes) starting at unit
// 16 J w.  Lane (g, u) = (lane / 16, lane % 16) takes rows g + 4 i (i < I) and
// units u + 16 j (j < J) of the slice.
//   - Per wavefront, the activation slice (1 KB per J) is one 16-byte load per
//     lane and the slice's scales of all 4 I rows (32 J bytes a row) one
//     16-byte load on 8 I J lanes; both go through the wavefront's own LDS
//     area and come back in the layout the products use.  Each load
//     instruction costs the address unit the same time whatever its width, so
//     this halves the instructions a wavefront issues.  Only the wavefront
//     itself reads its area: no barrier before the products.
//   - Partial sums are reduced over the 16 lanes of a row, then across the
//     wavefronts in wavefront order through LDS.
// Rows past n repeat row n - 1 and are not stored.
constexpr int kGemvKsMaxWaves = 10;

template <int I, int J, bool ROUTED = false>
__global__ void __launch_bounds__(64 * kGemvKsMaxWaves) gemv_ks_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                      int64_t k, const uint8_t* __restrict__ packed,
                                                                      const uint8_t* __restrict__ scales,
                                                                      const float* __restrict__ tscale_p,
                                                                      uint16_t* __restrict__ y, GvRoute rt = GvRoute{}) {
  constexpr int RB = 4 * I;
  constexpr int SL = 8 * I * J;  // lanes that load scales: 2 J pieces of 16 bytes per row
  static_assert(SL <= 64, "scale pieces per wavefront");
  __shared__ uint4 xs[kGemvKsMaxWaves][64 * J];
  __shared__ uint4 ss[kGemvKsMaxWaves][64];  // slots SL .. 63 take the repeated pieces
  __shared__ float red[kGemvKsMaxWaves][RB];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int u = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * RB;
  const int64_t kh = k >> 1, kb = k >> 4;
  const int64_t ub = (int64_t)w * 16 * J + u;  // this lane's first unit
  {
    const GvRow rr = gv_resolve<ROUTED>(rt, x, y, k, n, packed, scales, tscale_p);
    y = rr.y;
    if (!rr.ok) {  // uniform per workgroup
      if (threadIdx.x < RB && row0 + threadIdx.x < n) y[row0 + threadIdx.x] = 0;
      return;
    }
    x = rr.x;
    packed = rr.packed;
    scales = rr.scales;
    tscale_p = rr.tscale;
  }

  // 1. activations: piece 64 j + lane of the slice (8 elements)
  const uint4* xsl = reinterpret_cast<const uint4*>(x + (int64_t)w * 512 * J);
  uint4 xg[J];
#pragma unroll
  for (int j = 0; j < J; ++j) xg[j] = xsl[64 * j + lane];
  // 2. scales: lane l takes piece l % (2 J) of row (l % SL) / (2 J); lanes
  //    past SL repeat a piece into spare slots (no branch, so the compiler
  //    neither sinks the load nor drains the loads in flight at a join)
  uint4 sg;
  {
    const int sp = lane % SL;
    const int64_t r = row0 + sp / (2 * J), row = r < n ? r : n - 1;
    // plain load: 32 bytes of a line whose rest the other wavefronts read
    sg = reinterpret_cast<const uint4*>(scales + row * kb + (int64_t)w * 32 * J)[sp % (2 * J)];
  }
  __builtin_amdgcn_sched_barrier(0);  // activations and scales are issued before the weights
  // 3. weights
  uint4 wv[J][I];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const int64_t r = row0 + g + 4 * i, row = r < n ? r : n - 1;
      wv[j][i] = ld_stream16(packed + row * kh + (ub + 16 * j) * 16);
    }
  __builtin_amdgcn_sched_barrier(0);
  // 4. through this wavefront's LDS area: activation piece q of unit v of
  //    slice part j sits at 64 j + 16 q + v (conflict-free reads below)
#pragma unroll
  for (int j = 0; j < J; ++j) xs[w][64 * j + 16 * (lane & 3) + (lane >> 2)] = xg[j];
  ss[w][lane] = sg;
  wave_lds_sync();
  uint4 xv[J][4];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[j][q] = xs[w][64 * j + 16 * q + u];
  const uint16_t* srow = reinterpret_cast<const uint16_t*>(&ss[w][0]);

  float acc[I];
#pragma unroll
  for (int i = 0; i < I; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const float2 sc = e4m3x2_to_f32<false>(srow[(g + 4 * i) * 16 * J + 16 * j + u]);
      float p0 = dot8(wv[j][i].x, xv[j][0], 0.0f);
      p0 = dot8(wv[j][i].y, xv[j][1], p0);
      float p1 = dot8(wv[j][i].z, xv[j][2], 0.0f);
      p1 = dot8(wv[j][i].w, xv[j][3], p1);
      acc[i] = fmaf(p0, sc.x, acc[i]);
      acc[i] = fmaf(p1, sc.y, acc[i]);
    }
#pragma unroll
  for (int i = 0; i < I; ++i) {
    const float v = group_sum<16>(acc[i]);
    if (u == 0) red[w][g + 4 * i] = v;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < RB && row0 + t < n) {
    float v = red[0][t];
    for (int ww = 1; ww < nw; ++ww) v += red[ww][t];
    y[row0 + t] = (uint16_t)f32_to_bf16_rne(v * *tscale_p);
  }
}

// Long K (k a multiple of 512, more than 10 slices of 512): the same product
// with W <= 16 wavefronts, slice s going to wavefront s % W, so each wavefront
// owns up to S slices (w, w + W, ...).  Every load of all its slices is issued
// first (a slice past the end repeats the last one, in bounds, and its products
// are dropped by a select); then the slices are staged through the
// wavefront's LDS area one after another and accumulated in slice order.
// Slice i of a wavefront's share in gemv_ksl_kernel, then the next one: the
// activation piece and the scale pieces through the wavefront's LDS area, the
// products of its I rows added to acc when the slice exists.
typedef uint32_t ksl_u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ksl_u4(ksl_u32x4_t v) { return make_uint4(v.x, v.y, v.z, v.w); }

template <int I, int S, int i>
__device__ __forceinline__ void ksl_slices(const ksl_u32x4_t (&xg)[S], const ksl_u32x4_t (&sg)[S],
                                           const ksl_u32x4_t (&wv)[S][I], float (&acc)[I], uint4* xs, uint4* ss,
                                           int lane, int w, int nw, int nsl) {
  if constexpr (i < S) {
    const int u = lane & 15, g = lane >> 4;
    xs[16 * (lane & 3) + (lane >> 2)] = ksl_u4(xg[i]);
    ss[lane] = ksl_u4(sg[i]);
    wave_lds_sync();
    uint4 xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = xs[16 * q + u];
    const uint16_t* srw = reinterpret_cast<const uint16_t*>(ss);
    const bool valid = w + nw * i < nsl;  // uniform per wavefront
#pragma unroll
    for (int ii = 0; ii < I; ++ii) {
      const float2 sc = e4m3x2_to_f32<false>(srw[(g + 4 * ii) * 16 + u]);
      float p0 = dot8(wv[i][ii].x, xv[0], 0.0f);
      p0 = dot8(wv[i][ii].y, xv[1], p0);
      float p1 = dot8(wv[i][ii].z, xv[2], 0.0f);
      p1 = dot8(wv[i][ii].w, xv[3], p1);
      const float a = fmaf(p1, sc.y, fmaf(p0, sc.x, acc[ii]));
      acc[ii] = valid ? a : acc[ii];  // a select, not a branch: no wait for the loads still in flight
    }
    wave_lds_sync();  // the area is rewritten for the next slice
    ksl_slices<I, S, i + 1>(xg, sg, wv, acc, xs, ss, lane, w, nw, nsl);
  }
}

template <int I, int S>
__global__ void __launch_bounds__(1024) gemv_ksl_kernel(const uint16_t* __restrict__ x, int64_t n, int64_t k,
                                                        const uint8_t* __restrict__ packed,
                                                        const uint8_t* __restrict__ scales,
                                                        const float* __restrict__ tscale_p,
                                                        uint16_t* __restrict__ y) {
  constexpr int RB = 4 * I;
  constexpr int SL = 8 * I;  // lanes that load scales: 2 pieces of 16 bytes per row and slice
  static_assert(SL <= 64, "scale pieces per wavefront");
  __shared__ uint4 xs[16][64];
  __shared__ uint4 ss[16][64];
  __shared__ float red[16][RB];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int u = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * RB;
  const int64_t kh = k >> 1, kb = k >> 4;
  const int nsl = (int)(k >> 9);
  x += (int64_t)blockIdx.y * k;
  y += (int64_t)blockIdx.y * n;

  int sl[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int s = w + nw * i;
    sl[i] = s < nsl ? s : nsl - 1;
  }
  ksl_u32x4_t xg[S], sg[S];
  const int sp = lane % SL;
  const int64_t sr = row0 + sp / 2, srow = sr < n ? sr : n - 1;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    xg[i] = reinterpret_cast<const ksl_u32x4_t*>(x + (int64_t)sl[i] * 512)[lane];
    sg[i] = reinterpret_cast<const ksl_u32x4_t*>(scales + srow * kb + (int64_t)sl[i] * 32)[sp % 2];
  }
  __builtin_amdgcn_sched_barrier(0);  // activations and scales are issued before the weights
  ksl_u32x4_t wv[S][I];
#pragma unroll
  for (int i = 0; i < S; ++i)
#pragma unroll
    for (int ii = 0; ii < I; ++ii) {
      const int64_t r = row0 + g + 4 * ii, row = r < n ? r : n - 1;
      const uint4 v = ld_stream16(packed + row * kh + ((int64_t)sl[i] * 16 + u) * 16);
      wv[i][ii] = ksl_u32x4_t{v.x, v.y, v.z, v.w};
    }
  __builtin_amdgcn_sched_barrier(0);

  float acc[I];
#pragma unroll
  for (int ii = 0; ii < I; ++ii) acc[ii] = 0.0f;
  // Slices in order, each index a constant (a loop here, with its wavefront
  // barriers, stays rolled and puts the register arrays in scratch memory).
  ksl_slices<I, S, 0>(xg, sg, wv, acc, xs[w], ss[w], lane, w, nw, nsl);
#pragma unroll
  for (int ii = 0; ii < I; ++ii) {
    const float v = group_sum<16>(acc[ii]);
    if (u == 0) red[w][g + 4 * ii] = v;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < RB && row0 + t < n) {
    float v = red[0][t];
    for (int ww = 1; ww < nw; ++ww) v += red[ww][t];
    y[row0 + t] = (uint16_t)f32_to_bf16_rne(v * *tscale_p);
  }
}

template <int I, int S>
static void launch_ksl_rows(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                            const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
  const unsigned gx = (unsigned)((n + 4 * I - 1) / (4 * I));
  const int nsl = (int)(k >> 9), waves = (nsl + S - 1) / S;  // the fewest wavefronts with S slices each
  const int64_t max_y = 65535;
  for (int64_t m0 = 0; m0 < m; m0 += max_y) {
    const unsigned gy = (unsigned)((m - m0) < max_y ? (m - m0) : max_y);
    gemv_ksl_kernel<I, S><<<dim3(gx, gy), 64 * waves, 0, s>>>(x + m0 * k, n, k, packed, scales, tscale,
                                                                y + m0 * n);
  }
}

// 10 < k / 512 <= 64: S = ceil(slices / 16) slices per wavefront on the fewest
// wavefronts that cover them (5120 x 17408: 34 slices, 12 wavefronts of 3, 427
// workgroups of 12 rows), measured against the alternatives at that shape:
// 11.8 us; sixteen wavefronts (two to three slices each, 14 of them loading a
// repeated slice) 14.6 us; 8 rows per workgroup 12.1 us, 16 rows 14.8 us; the
// row-per-wavefront loop kernel it replaced 15.7 us.
static void launch_ksl(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                       const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
  switch ((int)((k >> 9) + 15) / 16) {
    case 1: return launch_ksl_rows<3, 1>(x, m, n, k, packed, scales, tscale, y, s);
    case 2: return launch_ksl_rows<3, 2>(x, m, n, k, packed, scales, tscale, y, s);
    case 3: return launch_ksl_rows<3, 3>(x, m, n, k, packed, scales, tscale, y, s);
    default: return launch_ksl_rows<3, 4>(x, m, n, k, packed, scales, tscale, y, s);
  }
}

// waves = k / 512 (one 512-element slice per wavefront).
template <int I>
static void launch_ks_rows(const uint16_t* x, int64_t m, int64_t n, int64_t k, int waves, const uint8_t* packed,
                           const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
  const unsigned gx = (unsigned)((n + 4 * I - 1) / (4 * I));
  const int64_t max_y = 65535;
  for (int64_t m0 = 0; m0 < m; m0 += max_y) {
    const unsigned gy = (unsigned)((m - m0) < max_y ? (m - m0) : max_y);
    gemv_ks_kernel<I, 1><<<dim3(gx, gy), 64 * waves, 0, s>>>(x + m0 * k, n, k, packed, scales, tscale, y + m0 * n);
  }
}

// Rows per workgroup, measured at k = 5120 (10 wavefronts): 12 rows for n up to
// 8192 (n = 5120: 427 workgroups, 5.51 us against 5.60 us with 20 rows and 6.32 us
// with 16), 16 rows above (n = 34816: 18.2 us against 19.0 us with 20 rows and
// 18.6 us with 12).  Fewer rows per workgroup give more workgroups to spread over
// the CUs, more rows give each wavefront more loads in flight.
static void launch_ks(const uint16_t* x, int64_t m, int64_t n, int64_t k, int waves, const uint8_t* packed,
                      const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
  if (n <= 8192) return launch_ks_rows<3>(x, m, n, k, waves, packed, scales, tscale, y, s);
  launch_ks_rows<4>(x, m, n, k, waves, packed, scales, tscale, y, s);
}

template <int LPR, int R, int JB, int W, bool RAGGED = false>
static void launch_lds(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                       const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
  constexpr int64_t rows_per_block = (int64_t)W * R * (64 / LPR);
  const unsigned gx = (unsigned)((n + rows_per_block - 1) / rows_per_block);
  const int64_t max_y = 65535;
  for (int64_t m0 = 0; m0 < m; m0 += max_y) {
    const unsigned gy = (unsigned)((m - m0) < max_y ? (m - m0) : max_y);
    gemv_lds_kernel<LPR, R, JB, W, RAGGED><<<dim3(gx, gy), 64 * W, 0, s>>>(x + m0 * k, n, k, packed, scales, tscale,
                                                                          y + m0 * n);
  }
}

// Dispatch for the LDS kernel: 32 lanes per row when k / 32 splits evenly into
// at most 8 units per lane, else 64 lanes per row with a ragged last unit.
// Rows per workgroup: 20 (10 wavefronts x 2 rows) for moderate n, so that a
// 5120-row weight maps onto exactly one workgroup per CU; 32 (8 x 2 x 2) for large n.
template <int LPR, int JB, bool RAGGED>
static void launch_lds_for_n(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                             const uint8_t* scales, const float* tscale, uint16_t* y, hipStream_t s) {
  if (n >= 16384)
    launch_lds<LPR, 2, JB, 8, RAGGED>(x, m, n, k, packed, scales, tscale, y, s);
  else
    launch_lds<LPR, 1, JB, 10, RAGGED>(x, m, n, k, packed, scales, tscale, y, s);
}

void launch_gemv_routed(const uint16_t* x, int64_t t_count, int64_t topk, const int32_t* route, int64_t experts,
                        int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales, const float* tscale,
                        uint16_t* y, hipStream_t s) {
  const int64_t pairs = t_count * topk, max_y = 65535;
  for (int64_t p0 = 0; p0 < pairs; p0 += max_y) {
    const unsigned gy = (unsigned)((pairs - p0) < max_y ? (pairs - p0) : max_y);
    const GvRoute rt{route, topk, experts, p0, n * (k >> 1)};
    if ((k & 511) == 0 && (k >> 9) <= kGemvKsMaxWaves) {
      // Rows per workgroup as for the dense call (top-8 of 128 experts of
      // 2048 x 4096, one token: 8.97 us with 12 rows against 9.34 with 16 and
      // 9.8 with 20).
      const unsigned w = 64 * (unsigned)(k >> 9);
      if (n <= 8192)
        gemv_ks_kernel<3, 1, true><<<dim3((unsigned)((n + 11) / 12), gy), w, 0, s>>>(x, n, k, packed, scales, tscale,
                                                                                      y, rt);
      else
        gemv_ks_kernel<4, 1, true><<<dim3((unsigned)((n + 15) / 16), gy), w, 0, s>>>(x, n, k, packed, scales, tscale,
                                                                                      y, rt);
    } else {
      const unsigned gx = (unsigned)((n + kGemvWaves * 2 - 1) / (kGemvWaves * 2));
      if ((k & 31) == 0)
        gemv_loop_kernel<2, 1, 2, true><<<dim3(gx, gy), kGemvThreads, 0, s>>>(x, n, k, packed, scales, tscale, y, rt);
      else
        gemv_loop_kernel<2, 1, 1, true><<<dim3(gx, gy), kGemvThreads, 0, s>>>(x, n, k, packed, scales, tscale, y, rt);
    }
  }
}

void launch_gemv(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                 const float* tscale, uint16_t* y, hipStream_t s) {
  if ((k & 511) == 0 && (k >> 9) <= kGemvKsMaxWaves)
    return launch_ks(x, m, n, k, (int)(k >> 9), packed, scales, tscale, y, s);
  if ((k & 511) == 0 && (k >> 9) <= 64) return launch_ksl(x, m, n, k, packed, scales, tscale, y, s);
  const int64_t units = k >> 5;
  if ((k & 31) == 0 && k <= kLdsMaxK) {
    if (units % 32 == 0) {
      switch (units / 32) {
        case 1: return launch_lds_for_n<32, 1, false>(x, m, n, k, packed, scales, tscale, y, s);
        case 2: return launch_lds_for_n<32, 2, false>(x, m, n, k, packed, scales, tscale, y, s);
        case 3: return launch_lds_for_n<32, 3, false>(x, m, n, k, packed, scales, tscale, y, s);
        case 4: return launch_lds_for_n<32, 4, false>(x, m, n, k, packed, scales, tscale, y, s);
        case 5: return launch_lds_for_n<32, 5, false>(x, m, n, k, packed, scales, tscale, y, s);
        case 6: return launch_lds_for_n<32, 6, false>(x, m, n, k, packed, scales, tscale, y, s);
        case 7: return launch_lds_for_n<32, 7, false>(x, m, n, k, packed, scales, tscale, y, s);
        case 8: return launch_lds_for_n<32, 8, false>(x, m, n, k, packed, scales, tscale, y, s);
        default: break;
      }
    } else if (units < 32) {
      return launch_lds_for_n<16, 2, true>(x, m, n, k, packed, scales, tscale, y, s);
    } else {
      switch ((units + 63) / 64) {
        case 1: return launch_lds_for_n<64, 1, true>(x, m, n, k, packed, scales, tscale, y, s);
        case 2: return launch_lds_for_n<64, 2, true>(x, m, n, k, packed, scales, tscale, y, s);
        case 3: return launch_lds_for_n<64, 3, true>(x, m, n, k, packed, scales, tscale, y, s);
        case 4: return launch_lds_for_n<64, 4, true>(x, m, n, k, packed, scales, tscale, y, s);
        default: break;
      }
    }
  }
  launch_rj<2, 1>(x, m, n, k, packed, scales, tscale, y, s);
}

}  // namespace nvfp4
