// Quantizer (BF16 -> NVFP4) and dequantizer kernels for gfx950.
//
// The quantizer is imp-quantize's round-to-nearest scheme (imp
// "docs/quantization.md", imp-quantize section: plain round-to-nearest scales
// over the weights, no calibration; the micro-scale paragraph: the scale is
// taken from the block absmax, and the FP4 grid is 0, 0.5, 1, 1.5, 2, 3, 4, 6):
//   tscale = fl32(amax / 2688)
//   scale  = E4M3 code nearest to 448 * bam / amax           (ties to even)
//   code   = sign(w) | E2M1 code nearest to 2688 |w| / (amax s)   (ties to even, saturating)
// Each rounding is the hardware's nearest-even conversion of an FP32 value
// that equals the exact quotient at a midpoint and lies on the exact
// quotient's side of every midpoint otherwise, so the result is the decision
// on the exact real quotients.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// amax: max |w| over the tensor.  The maximum of BF16 magnitudes is taken on
// their bit patterns (bits & 0x7FFF order like the values), so it is exact
// and independent of the order.  Each thread keeps kAmaxU 16-byte loads in
// flight; a workgroup reduces to one value, which goes either to a partial
// slot (reduced by one more workgroup) or, to merge into a caller's running
// maximum, through an unsigned atomic max on the FP32 bit pattern.  Same-
// address atomics serialise, so the atomic form uses few workgroups.
// ---------------------------------------------------------------------------
constexpr int kAmaxU = 8;
constexpr int kAmaxBlocks = 512;          // atomic form
constexpr int kAmaxPartialBlocks = 8192;  // partial-slot form: one pass over the data per thread
constexpr int kAmaxSharedParts = 1024;    // form whose maxima every encode workgroup reduces (4 per thread)

typedef unsigned short amax_u16x2_t __attribute__((ext_vector_type(2)));

// Lane-wise 16-bit maxima of the magnitude bits of 8 BF16 (two per 32 bits).
__device__ __forceinline__ amax_u16x2_t bf16x8_absmax_pair(uint4 v) {
  const auto m = [](uint32_t x) { return __builtin_bit_cast(amax_u16x2_t, x & 0x7FFF7FFFu); };
  return __builtin_elementwise_max(__builtin_elementwise_max(m(v.x), m(v.y)), __builtin_elementwise_max(m(v.z), m(v.w)));
}

// The workgroup's maximum |w| (BF16 magnitude bits), valid in thread 0.
// Loads never branch: an index past the end loads the last vector again, which
// cannot change the maximum.
__device__ __forceinline__ uint32_t amax_block(const uint4* __restrict__ w, int64_t n_vec) {
  amax_u16x2_t mp = {0, 0};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * kAmaxU;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x * kAmaxU + threadIdx.x; i0 < n_vec; i0 += stride) {
    uint4 v[kAmaxU];
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) {
      const int64_t i = i0 + (int64_t)u * blockDim.x;
      // Plain loads: the encode pass reads w again (with the nontemporal hint
      // the quantizer took 26.3 us instead of 24.9 at 5120 x 5120).
      v[u] = w[i < n_vec ? i : n_vec - 1];
    }
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) mp = __builtin_elementwise_max(mp, bf16x8_absmax_pair(v[u]));
  }
  uint32_t m = max((uint32_t)mp[0], (uint32_t)mp[1]);
  m = wave_max_u32(m);
  __shared__ uint32_t part[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) part[wid] = m;
  __syncthreads();
  uint32_t r = part[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = max(r, part[i]);
  return r;
}

// Per-workgroup maxima into part[blockIdx.x] (BF16 magnitude bits).  Over a
// stack of matrices, blockIdx.y picks the matrix: w_stride 16-byte vectors and
// part_stride words apart.
__global__ void __launch_bounds__(256) amax_partial_kernel(const uint4* __restrict__ w, int64_t n_vec,
                                                           uint32_t* __restrict__ part, int64_t w_stride,
                                                           int64_t part_stride) {
  const uint32_t r = amax_block(w + (int64_t)blockIdx.y * w_stride, n_vec);
  if (threadIdx.x == 0) part[(int64_t)blockIdx.y * part_stride + blockIdx.x] = r;
}

// amax[y] = max of part[y][0 .. nb) as an FP32 value (the BF16 magnitude
// widened); y = blockIdx.y over a stack.  With TSCALE the value written is the
// tensor scale fl32(amax / 2688) instead (the quantize pass then recovers amax
// from it exactly, see amax_bits_from_tscale).
template <bool TSCALE>
__global__ void __launch_bounds__(256) amax_reduce_kernel(const uint32_t* __restrict__ part, int nb, float* amax,
                                                          int64_t part_stride) {
  part += (int64_t)blockIdx.y * part_stride;
  amax += blockIdx.y;
  // Eight independent loads per thread in flight (one pass for nb <= 2048).
  uint32_t mv[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  for (int i0 = threadIdx.x; i0 < nb; i0 += blockDim.x * 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * (int)blockDim.x;
      mv[u] = max(mv[u], part[i < nb ? i : nb - 1]);  // a repeated slot cannot change the maximum
    }
  }
  uint32_t m = max(max(max(mv[0], mv[1]), max(mv[2], mv[3])), max(max(mv[4], mv[5]), max(mv[6], mv[7])));
  m = wave_max_u32(m);
  __shared__ uint32_t pw[4];
  if ((threadIdx.x & 63) == 0) pw[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float a = __uint_as_float(max(max(pw[0], pw[1]), max(pw[2], pw[3])) << 16);
    *amax = TSCALE ? __fdiv_rn(a, 2688.0f) : a;
  }
}

// *amax = max(*amax, max |w|) through an atomic max on the FP32 bits.
__global__ void __launch_bounds__(256) amax_kernel(const uint4* __restrict__ w, int64_t n_vec, float* amax) {
  const uint32_t r = amax_block(w, n_vec);
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(amax), r << 16);  // BF16 magnitude -> FP32 bits
}

// tscale = fl32(amax / 2688), IEEE round-to-nearest division; one value per
// thread over a stack of n matrices.
__global__ void __launch_bounds__(64) finalize_tscale_kernel(const float* amax, float* tscale, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) tscale[i] = __fdiv_rn(amax[i], 2688.0f);
}

// ---------------------------------------------------------------------------
// Quantize.
// ---------------------------------------------------------------------------

// BF16 bits of amax from its tensor scale t = fl32(amax / 2688): the BF16
// value nearest to fl32(2688 t) is amax again, for every finite non-negative
// BF16 amax (FP32 subnormal t included; 2688 t is within a relative 2^-23 of
// amax, far closer than half a BF16 step).
__device__ __forceinline__ uint32_t amax_bits_from_tscale(float t) { return f32_to_bf16_rne(2688.0f * t); }

// Rounding decisions through FP64 and the gfx950 conversion instructions.
//
// Both roundings of the quantizer are "nearest grid point of an exact
// quotient, ties to the even code": the E4M3 scale of 448 bam / amax and the
// E2M1 magnitude of 2688 |w| / (amax s).  Every operand is a BF16 or E4M3
// value (at most 8 significant bits), so when such a quotient is not exactly a
// midpoint of its grid it lies at least a relative 2^-17 away from every
// midpoint (numerator and denominator are small integers times powers of two:
// a nonzero difference is at least the smaller power of two).  The quotient is
// formed in FP64 from one correctly rounded division and one product (relative
// error below 2^-51), then rounded to FP32: a midpoint (a short FP32 value)
// comes out exactly, and every other quotient stays on its side of every
// midpoint.  The hardware FP32 -> E4M3 / E2M1 conversions round to nearest
// even on the exact FP32 input, which is then the decision on the exact real
// quotient.  E2M1 saturates at 6 (code 7), as the nearest-code rule does.

// The E4M3 code nearest to r, 0 <= r <= 448 (hardware conversion, round to
// nearest even, OCP E4M3FN).
__device__ __forceinline__ uint32_t e4m3_code_rne(float r) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r, 0.0f, 0, false) & 0xFFu;
}

// Per-tensor constants: k448 = 448 / amax and k2688 = 2688 / amax in FP64
// (correctly rounded divisions); zero when amax is 0 (then every scale and code
// is 0).
struct QuantConsts {
  double k448, k2688;
};

__device__ __forceinline__ QuantConsts quant_consts(uint32_t amax_b) {
  const double a = (double)__uint_as_float((amax_b & 0x7FFFu) << 16);
  QuantConsts c;
  c.k448 = a > 0.0 ? 448.0 / a : 0.0;
  c.k2688 = a > 0.0 ? 2688.0 / a : 0.0;
  return c;
}

// Eight elements (one uint4 of BF16) to eight 4-bit codes in one word (element
// i in nibble i): code = E2M1 nearest to w * cq with the sign of w, where
// cq = 2688 / (amax s) in FP64 (0 for a zero scale: every magnitude code 0).
template <int J>
__device__ __forceinline__ uint32_t pair_codes(uint32_t word, uint32_t e, double cq) {
  const float lo = (float)((double)__uint_as_float(e << 16) * cq);
  const float hi = (float)((double)__uint_as_float(e & 0xFFFF0000u) * cq);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, lo, hi, 1.0f, J);
}

__device__ __forceinline__ uint32_t half_codes(const uint4 v, double cq) {
  uint32_t word = pair_codes<0>(0u, v.x, cq);
  word = pair_codes<1>(word, v.y, cq);
  word = pair_codes<2>(word, v.z, cq);
  return pair_codes<3>(word, v.w, cq);
}

// One thread per 16-element block at a time: two 16-byte loads (8 BF16 each),
// one 64-bit store of the 16 codes, one scale byte.  Each thread loads
// kQuantB blocks (blockDim apart) before it encodes any of them.
constexpr int kQuantB = 2;

struct BlockCodes {
  uint32_t lo, hi, scode;  // codes of elements 0..7 and 8..15, scale code
};

// Largest magnitude (bits & 0x7FFF) of 8 BF16, by lane-wise 16-bit maxima.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2_t mag2(uint32_t x) { return __builtin_bit_cast(u16x2_t, x & 0x7FFF7FFFu); }

__device__ __forceinline__ uint32_t half_max(const uint4 v) {
  const u16x2_t a = __builtin_elementwise_max(__builtin_elementwise_max(mag2(v.x), mag2(v.y)),
                                              __builtin_elementwise_max(mag2(v.z), mag2(v.w)));
  return max((uint32_t)a[0], (uint32_t)a[1]);
}

__device__ __forceinline__ BlockCodes quantize_block(const uint4 v0, const uint4 v1, const QuantConsts& c) {
  const uint32_t bam = max(half_max(v0), half_max(v1));
  // Scale: E4M3 nearest to 448 bam / amax (at most 448: bam <= amax).
  const float r = (float)((double)__uint_as_float(bam << 16) * c.k448);
  const uint32_t scode = e4m3_code_rne(fminf(r, 448.0f));
  // Elements: E2M1 nearest to 2688 |w| / (amax s), s the E4M3 value of scode.
  const double s = (double)e4m3x2_to_f32<false>(scode).x;
  const double cq = scode ? c.k2688 / s : 0.0;
  return BlockCodes{half_codes(v0, cq), half_codes(v1, cq), scode};
}

// 8 codes (one 32-bit word) decoded to E2M1 * E4M3 (no tensor scale) as 8 BF16.
// Each product has at most 6 significant bits, so it is exact in FP32 and its
// upper 16 bits are the exact BF16 value (signed zeros kept).
__device__ __forceinline__ uint32_t decode_pair_bf16(float2 v, float s) {
  return (__float_as_uint(v.x * s) >> 16) | (__float_as_uint(v.y * s) & 0xFFFF0000u);
}

template <int SEL>
__device__ __forceinline__ float2 e2m1_pair(uint32_t word) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
  return make_float2(v[0], v[1]);
}

__device__ __forceinline__ uint4 decode_half_bf16(uint32_t word, uint32_t scode) {
  const float s = e4m3x2_to_f32<false>(scode).x;
  return make_uint4(decode_pair_bf16(e2m1_pair<0>(word), s), decode_pair_bf16(e2m1_pair<1>(word), s),
                    decode_pair_bf16(e2m1_pair<2>(word), s), decode_pair_bf16(e2m1_pair<3>(word), s));
}

template <bool DECODE>
__device__ __forceinline__ void store_block(int64_t blk, BlockCodes q, uint2* __restrict__ packed,
                                            uint8_t* __restrict__ scales, uint4* __restrict__ decoded) {
  packed[blk] = make_uint2(q.lo, q.hi);
  scales[blk] = (uint8_t)q.scode;
  if constexpr (DECODE) {
    decoded[2 * blk] = decode_half_bf16(q.lo, q.scode);
    decoded[2 * blk + 1] = decode_half_bf16(q.hi, q.scode);
  }
}

// Where the encode pass takes amax from.
enum AmaxSrc : int {
  kFromAmax = 0,    // amax_p: amax (a BF16 value held in FP32)
  kFromTscale = 1,  // amax_p: the tensor scale, amax recovered from it
  kFromParts = 2,   // parts[0 .. nparts): per-workgroup maxima (BF16 magnitude bits) that every workgroup
                    // reduces itself; workgroup 0 writes the tensor scale to ts_out
};

// Maximum of parts[0 .. nparts) (1 <= nparts <= 4 x 256) over a 256-thread
// workgroup; every thread receives it.  Indices past the end load the last
// slot again, which cannot change the maximum.
__device__ __forceinline__ uint32_t parts_max(const uint32_t* __restrict__ parts, int nparts) {
  uint32_t mv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = (int)threadIdx.x + 256 * u;
    mv[u] = parts[i < nparts ? i : nparts - 1];
  }
  uint32_t m = wave_max_u32(max(max(mv[0], mv[1]), max(mv[2], mv[3])));
  __shared__ uint32_t pw[4];
  if ((threadIdx.x & 63) == 0) pw[threadIdx.x >> 6] = m;
  __syncthreads();
  return max(max(pw[0], pw[1]), max(pw[2], pw[3]));
}

// The activation quantizer of the NVFP4 x NVFP4 linear: the encode pass that
// also writes each element's exact BF16 value E2M1 x E4M3 (DECODE of
// store_block), one thread per block.  Iterations whose kQuantB blocks all
// exist run without a branch between loads, codes and stores, so the compiler
// interleaves the blocks; only the grid's last iteration takes the guarded
// path.  One thread also writes ts_x = fl32(amax / 2688) and ts_y =
// fl32(ts_w * ts_x).  Every workgroup reads only amax_p, which is neither of
// them; the linear that follows reads ts_y.
__global__ void __launch_bounds__(256) quantize_decode_kernel(const uint4* __restrict__ w, int64_t n_blk,
                                                              const float* __restrict__ amax_p,
                                                              uint2* __restrict__ packed,
                                                              uint8_t* __restrict__ scales,
                                                              uint4* __restrict__ decoded, const float* ts_w,
                                                              float* ts_x, float* ts_y) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const float tx = __fdiv_rn(amax_p[0], 2688.0f);
    ts_x[0] = tx;
    ts_y[0] = ts_w[0] * tx;
  }
  // amax is a BF16 value held in FP32
  const QuantConsts qc = quant_consts(__float_as_uint(amax_p[0]) >> 16);
  const int64_t B = blockDim.x;
  const int64_t stride = (int64_t)gridDim.x * B * kQuantB;
  for (int64_t b0 = (int64_t)blockIdx.x * B * kQuantB + threadIdx.x; b0 < n_blk; b0 += stride) {
    uint4 v[2 * kQuantB];
    if (b0 + (kQuantB - 1) * B < n_blk) {
#pragma unroll
      for (int u = 0; u < kQuantB; ++u) {
        // Plain loads: an instruction reads half lines (32-byte stride), and
        // the nontemporal hint made the line's other half miss again.
        v[2 * u] = w[2 * (b0 + u * B)];
        v[2 * u + 1] = w[2 * (b0 + u * B) + 1];
      }
      BlockCodes q[kQuantB];
#pragma unroll
      for (int u = 0; u < kQuantB; ++u) q[u] = quantize_block(v[2 * u], v[2 * u + 1], qc);
#pragma unroll
      for (int u = 0; u < kQuantB; ++u) store_block<true>(b0 + u * B, q[u], packed, scales, decoded);
    } else {
#pragma unroll
      for (int u = 0; u < kQuantB; ++u) {
        const int64_t blk = b0 + u * B;
        if (blk < n_blk) {
          store_block<true>(blk, quantize_block(w[2 * blk], w[2 * blk + 1], qc), packed, scales, decoded);
        }
      }
    }
  }
}

// The encode pass (without the BF16 decode) with whole-line loads.  A
// wavefront takes 64 kQuantB consecutive blocks per iteration (4 KiB of W):
// load instruction j brings vector 64 j + lane of that range (1 KiB of
// contiguous lines), the vectors go through the wavefront's own LDS area, and
// lane l reads back the two vectors of block 64 u + l.  Only the wavefront
// uses its area, so a wavefront-scope synchronization (wave_lds_sync) is all
// it needs.  The stores are as above (8 bytes of codes and one scale byte per
// lane and block, consecutive lanes on consecutive blocks).
template <int SRC>
__global__ void __launch_bounds__(256) quantize_lines_kernel(const uint4* __restrict__ w, int64_t n_blk,
                                                             const float* __restrict__ amax_p,
                                                             uint2* __restrict__ packed,
                                                             uint8_t* __restrict__ scales,
                                                             const uint32_t* __restrict__ parts, int nparts,
                                                             float* ts_out) {
  constexpr int V = 2 * kQuantB;  // vectors per lane and iteration
  __shared__ uint4 area[4][64 * V];
  w += (int64_t)blockIdx.y * 2 * n_blk;
  packed += (int64_t)blockIdx.y * n_blk;
  scales += (int64_t)blockIdx.y * n_blk;
  uint32_t amax_b;
  if constexpr (SRC == kFromParts) {
    amax_b = parts_max(parts + (int64_t)blockIdx.y * nparts, nparts);
    if (blockIdx.x == 0 && threadIdx.x == 0) ts_out[blockIdx.y] = __fdiv_rn(__uint_as_float(amax_b << 16), 2688.0f);
  } else if constexpr (SRC == kFromTscale) {
    amax_b = amax_bits_from_tscale(amax_p[blockIdx.y]);
  } else {
    amax_b = __float_as_uint(amax_p[blockIdx.y]) >> 16;
  }
  const QuantConsts qc = quant_consts(amax_b);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint4* my = area[wv];
  const int64_t n_vec = 2 * n_blk;
  const int64_t chunk = 64 * kQuantB;  // blocks per wavefront and iteration
  const int64_t stride = (int64_t)gridDim.x * 4 * chunk;
  for (int64_t c0 = ((int64_t)blockIdx.x * 4 + wv) * chunk; c0 < n_blk; c0 += stride) {
    uint4 v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = 2 * c0 + 64 * j + lane;
      v[j] = w[i < n_vec ? i : n_vec - 1];  // past the end: an in-bounds load, never stored
    }
#pragma unroll
    for (int j = 0; j < V; ++j) my[64 * j + lane] = v[j];
    wave_lds_sync();
    BlockCodes q[kQuantB];
#pragma unroll
    for (int u = 0; u < kQuantB; ++u) q[u] = quantize_block(my[128 * u + 2 * lane], my[128 * u + 2 * lane + 1], qc);
    wave_lds_sync();  // the next iteration rewrites the area
#pragma unroll
    for (int u = 0; u < kQuantB; ++u) {
      const int64_t blk = c0 + 64 * u + lane;
      if (blk < n_blk) store_block<false>(blk, q[u], packed, scales, nullptr);
    }
  }
}

// ---------------------------------------------------------------------------
// Dequantize: w = RNE_bf16(fl32(fl32(E2M1 * E4M3) * tscale)).  One thread per
// 8 elements at a time: one packed word in, one uint4 (8 BF16) out; each
// thread loads kDequantU words (blockDim apart) before decoding them.
// ---------------------------------------------------------------------------
constexpr int kDequantU = 4;

__device__ __forceinline__ uint4 dequant_half(uint32_t p, uint32_t sbyte, float t) {
  return e2m1x8_dequant_bf16(p, e4m3x2_to_f32<false>(sbyte).x, t);
}

// Over a stack, blockIdx.y picks the matrix (n_half half blocks each).
__global__ void __launch_bounds__(256) dequant_kernel(const uint32_t* __restrict__ packed,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ tscale_p, int64_t n_half,
                                                      uint4* __restrict__ out) {
  packed += (int64_t)blockIdx.y * n_half;
  scales += (int64_t)blockIdx.y * (n_half >> 1);
  out += (int64_t)blockIdx.y * n_half;
  const float t = tscale_p[blockIdx.y];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * kDequantU;
  for (int64_t h0 = (int64_t)blockIdx.x * blockDim.x * kDequantU + threadIdx.x; h0 < n_half; h0 += stride) {
    // Loads never branch: an index past the end reads the last half block
    // again (its result is not stored), so every load is issued before any
    // wait.  Nontemporal stores: the BF16 weight is written once and not read
    // back here.
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    uint32_t p[kDequantU], sb[kDequantU];
#pragma unroll
    for (int u = 0; u < kDequantU; ++u) {
      const int64_t h = h0 + (int64_t)u * blockDim.x;
      const int64_t hc = h < n_half ? h : n_half - 1;
      // Plain loads: 4- and 1-byte lanes (with the nontemporal hint this pass
      // took 30 % longer).
      p[u] = packed[hc];
      sb[u] = scales[hc >> 1];
    }
#pragma unroll
    for (int u = 0; u < kDequantU; ++u) {
      const int64_t h = h0 + (int64_t)u * blockDim.x;
      if (h < n_half) {
        const uint4 v = dequant_half(p[u], sb[u], t);
        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(out) + h);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
static inline unsigned grid_for(int64_t items, int threads, int64_t max_blocks) {
  int64_t b = (items + threads - 1) / threads;
  if (b > max_blocks) b = max_blocks;
  if (b < 1) b = 1;
  return (unsigned)b;
}

void launch_amax(const uint16_t* w, int64_t n_elems, float* amax, hipStream_t s) {
  const int64_t n_vec = n_elems / 8;
  amax_kernel<<<grid_for(n_vec, 256 * kAmaxU, kAmaxBlocks), 256, 0, s>>>(reinterpret_cast<const uint4*>(w), n_vec,
                                                                          amax);
}

void launch_amax_set(const uint16_t* w, int64_t n_elems, uint32_t* part, float* amax, hipStream_t s) {
  launch_amax_set_stack(w, 1, n_elems, part, amax, s);
}

void launch_amax_set_stack(const uint16_t* w, int64_t count, int64_t n_elems, uint32_t* part, float* amax,
                           hipStream_t s) {
  // Matrix i's partial maxima go to part + i * n_elems / 8: the packed output of matrix i (n_elems / 8 words), and
  // the grid never exceeds n_elems / 8 workgroups.
  const int64_t n_vec = n_elems / 8;
  const unsigned nb = grid_for(n_vec, 256 * kAmaxU, kAmaxPartialBlocks);
  amax_partial_kernel<<<dim3(nb, (unsigned)count), 256, 0, s>>>(reinterpret_cast<const uint4*>(w), n_vec, part, n_vec,
                                                                n_vec);
  amax_reduce_kernel<false><<<dim3(1, (unsigned)count), 256, 0, s>>>(part, (int)nb, amax, n_vec);
}

void launch_tscale_set_stack(const uint16_t* w, int64_t count, int64_t n_elems, uint32_t* part, float* tscale,
                             hipStream_t s) {
  const int64_t n_vec = n_elems / 8;
  const unsigned nb = grid_for(n_vec, 256 * kAmaxU, kAmaxPartialBlocks);
  amax_partial_kernel<<<dim3(nb, (unsigned)count), 256, 0, s>>>(reinterpret_cast<const uint4*>(w), n_vec, part, n_vec,
                                                                n_vec);
  amax_reduce_kernel<true><<<dim3(1, (unsigned)count), 256, 0, s>>>(part, (int)nb, tscale, n_vec);
}

void launch_quantize_shared_amax(const uint16_t* w, int64_t n_elems, uint32_t* parts, float* tscale,
                                 uint8_t* packed, uint8_t* scales, hipStream_t s) {
  const int64_t n_vec = n_elems / 8, n_blk = n_elems / 16;
  const unsigned nb = grid_for(n_vec, 256 * kAmaxU, kAmaxSharedParts);
  amax_partial_kernel<<<dim3(nb, 1u), 256, 0, s>>>(reinterpret_cast<const uint4*>(w), n_vec, parts, n_vec, n_vec);
  quantize_lines_kernel<kFromParts><<<dim3(grid_for(n_blk, 256 * kQuantB, 1 << 20), 1u), 256, 0, s>>>(
      reinterpret_cast<const uint4*>(w), n_blk, nullptr, reinterpret_cast<uint2*>(packed), scales, parts, (int)nb,
      tscale);
}

void launch_quantize_from_tscale(const uint16_t* w, int64_t count, int64_t n_elems, const float* tscale,
                                 uint8_t* packed, uint8_t* scales, hipStream_t s) {
  const int64_t n_blk = n_elems / 16;
  quantize_lines_kernel<kFromTscale>
      <<<dim3(grid_for(n_blk, 256 * kQuantB, 1 << 20), (unsigned)count), 256, 0, s>>>(
          reinterpret_cast<const uint4*>(w), n_blk, tscale, reinterpret_cast<uint2*>(packed), scales, nullptr, 0,
          nullptr);
}

void launch_finalize_tscale(const float* amax, float* tscale, int64_t count, hipStream_t s) {
  finalize_tscale_kernel<<<(unsigned)((count + 63) / 64), 64, 0, s>>>(amax, tscale, count);
}

void launch_quantize(const uint16_t* w, int64_t count, int64_t n_elems, const float* amax, uint8_t* packed,
                     uint8_t* scales, hipStream_t s) {
  const int64_t n_blk = n_elems / 16;
  quantize_lines_kernel<kFromAmax><<<dim3(grid_for(n_blk, 256 * kQuantB, 1 << 20), (unsigned)count), 256, 0, s>>>(
      reinterpret_cast<const uint4*>(w), n_blk, amax, reinterpret_cast<uint2*>(packed), scales, nullptr, 0, nullptr);
}

void launch_quantize_decode(const uint16_t* w, int64_t n_elems, const float* amax, uint8_t* packed, uint8_t* scales,
                            uint16_t* decoded, const float* ts_w, float* ts_x, float* ts_y, hipStream_t s) {
  const int64_t n_blk = n_elems / 16;
  quantize_decode_kernel<<<dim3(grid_for(n_blk, 256 * kQuantB, 1 << 20), 1u), 256, 0, s>>>(
      reinterpret_cast<const uint4*>(w), n_blk, amax, reinterpret_cast<uint2*>(packed), scales,
      reinterpret_cast<uint4*>(decoded), ts_w, ts_x, ts_y);
}

void launch_dequant(const uint8_t* packed, const uint8_t* scales, const float* tscale, int64_t count, int64_t n_elems,
                    uint16_t* out, hipStream_t s) {
  const int64_t n_half = n_elems / 8;
  dequant_kernel<<<dim3(grid_for(n_half, 256 * kDequantU, 1 << 20), (unsigned)count), 256, 0, s>>>(
      reinterpret_cast<const uint32_t*>(packed), scales, tscale, n_half, reinterpret_cast<uint4*>(out));
}

}  // namespace nvfp4
