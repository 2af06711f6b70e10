// Quantizer (BF16 -> NVFP4) and dequantizer kernels for gfx950.
//
// The quantizer is imp-quantize's round-to-nearest scheme (imp
// "docs/quantization.md", imp-quantize section: plain round-to-nearest scales
// over the weights, no calibration; the micro-scale paragraph: the scale is
// taken from the block absmax, and the FP4 grid is 0, 0.5, 1, 1.5, 2, 3, 4, 6):
//   tscale = fl32(amax / 2688)
//   scale  = E4M3 code nearest to 448 * bam / amax           (ties to even)
//   code   = sign(w) | E2M1 code nearest to 2688 |w| / (amax s)   (ties to even, saturating)
// Every decision compares two exact products in FP32 (operands are rescaled
// by powers of two so that both sides stay in range), so the result equals
// the decision on the exact real quotients.
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
constexpr int kAmaxBlocks = 512;

__device__ __forceinline__ uint32_t bf16x8_absmax_bits(uint4 v) {
  const uint32_t a = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  const uint32_t b = max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu));
  return max(a, b);
}

// The workgroup's maximum |w| (BF16 magnitude bits), valid in thread 0.
__device__ __forceinline__ uint32_t amax_block(const uint4* __restrict__ w, int64_t n_vec) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * kAmaxU;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x * kAmaxU + threadIdx.x; i0 < n_vec; i0 += stride) {
    uint4 v[kAmaxU];
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) {
      const int64_t i = i0 + (int64_t)u * blockDim.x;
      v[u] = i < n_vec ? w[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) m = max(m, bf16x8_absmax_bits(v[u]));
  }
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
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) m = max(m, part[i]);
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

// A finite BF16 magnitude b (bits & 0x7FFF) as sig * 2^ex with an integer sig < 256.
__device__ __forceinline__ void bf16_split(uint32_t b, uint32_t& sig, int& ex) {
  const uint32_t f = b >> 7;
  sig = (b & 0x7Fu) | (f ? 0x80u : 0u);
  ex = (f ? (int)f : 1) - 134;
}

// E4M3 value of a code as sig * 2^ex (sig <= 15).
__device__ __forceinline__ void e4m3_split(uint32_t c, uint32_t& sig, int& ex) {
  const uint32_t e = c >> 3, m = c & 7u;
  sig = e ? (8u + m) : m;
  ex = e ? (int)e - 10 : -9;
}

// Round a non-negative float to an E4M3 code (RNE), clamped to 0..126.  Used
// only for a first guess from an approximate quotient; the caller corrects it.
// Branch-free (selects), so that several blocks' searches can interleave.
__device__ __forceinline__ uint32_t e4m3_code_guess(float r) {
  uint32_t u = __float_as_uint(r);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  uint32_t c = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);   // normal range [2^-6, 448)
  c = c > 126u ? 126u : c;
  const uint32_t sub = (uint32_t)__builtin_rintf(r * 512.0f);  // subnormal range: multiples of 2^-9
  c = r < 0x1p-6f ? sub : c;
  return r < 448.0f ? c : 126u;                                // also NaN
}

// The E4M3 code nearest to 448 * bam / amax (ties to the even code).
// bam = sb * 2^eb, amax = sa * 2^ea.  With A = 448 sb 2^(eb-ea) and D = sa the
// quotient is A / D; the comparisons A vs u * D against the midpoints u are
// exact (u has <= 5 significant bits, D <= 8, A <= 17).  The guess is off by at
// most one code; one step up, then one step down, settles it.
__device__ __forceinline__ uint32_t e4m3_scale_code(uint32_t bam_b, uint32_t sa, int ea) {
  uint32_t sb;
  int eb;
  bf16_split(bam_b, sb, eb);
  const float A = ldexpf((float)(448u * sb), eb - ea);
  const float D = (float)sa;
  uint32_t c = e4m3_code_guess(A * __builtin_amdgcn_rcpf(D));
  // Neighbouring codes as one 16-bit pair, decoded by the hardware E4M3 conversion
  // (exact for every code; codes here are at most 126, never NaN).
  const uint32_t cu = c < 125u ? c : 125u;
  const auto pu = __builtin_amdgcn_cvt_pk_f32_fp8((int)(cu | ((cu + 1u) << 8)), false);
  const float up_rhs = 0.5f * (pu[0] + pu[1]) * D;
  // Bitwise forms of the tie rule (an odd code's upper midpoint rounds up), so
  // that no branch splits the block.
  const uint32_t odd_u = c & 1u;
  c += (uint32_t)(c < 126u) & ((odd_u & (uint32_t)(A >= up_rhs)) | ((odd_u ^ 1u) & (uint32_t)(A > up_rhs)));
  const uint32_t cd = c > 1u ? c : 1u;
  const auto pd = __builtin_amdgcn_cvt_pk_f32_fp8((int)((cd - 1u) | (cd << 8)), false);
  const float dn_rhs = 0.5f * (pd[0] + pd[1]) * D;
  const uint32_t odd_d = (c - 1u) & 1u;
  c -= (uint32_t)(c > 0u) & ((odd_d & (uint32_t)(A < dn_rhs)) | ((odd_d ^ 1u) & (uint32_t)(A <= dn_rhs)));
  return bam_b == 0u ? 0u : c;
}

// Per-block element thresholds.  With t_j = T_j / 4 the E2M1 midpoints
// (T = 1, 3, 5, 7, 10, 14, 20), the element decision 2688 |w| vs t_j amax s
// becomes  L = 21 |w| 2^(9 - ea - es)  vs  R_j = T_j sa ss  (2688 = 21 * 2^7).
struct ElemThresholds {
  float r[7];
  uint32_t u[7];  // bits of r
  int shift;      // 9 - ea - es
};

__device__ __forceinline__ ElemThresholds element_thresholds(uint32_t scode, uint32_t sa, int ea) {
  ElemThresholds t;
  uint32_t ss;
  int es;
  e4m3_split(scode, ss, es);
  // scale 0: every magnitude is 0 (compare against +inf)
  const float S = scode ? (float)(sa * ss) : __builtin_huge_valf();
  t.r[0] = 1.0f * S;
  t.r[1] = 3.0f * S;
  t.r[2] = 5.0f * S;
  t.r[3] = 7.0f * S;
  t.r[4] = 10.0f * S;
  t.r[5] = 14.0f * S;
  t.r[6] = 20.0f * S;
#pragma unroll
  for (int j = 0; j < 7; ++j) t.u[j] = __float_as_uint(t.r[j]);
  t.shift = 9 - ea - es;
  return t;
}

// 4-bit code of one BF16 element (bits in the low 16 bits of b).
// The magnitude code is the number of midpoints L passes (ties to the even
// code: L must reach an odd code's upper midpoint R_1, R_3, R_5 and exceed an
// even code's R_0, R_2, R_4, R_6).  The R_j increase with j, so a binary search
// takes three of the seven exact comparisons: R_3, then R_5 or R_1, then the
// even midpoint just below.
__device__ __forceinline__ uint32_t element_code(uint32_t b, const ElemThresholds& t) {
  // Selects are written as bit masks so that they stay v_cndmask / v_bfi and
  // never become branches.
  const float L = 21.0f * ldexpf(__uint_as_float((b & 0x7FFFu) << 16), t.shift);
  const uint32_t hi = 0u - (uint32_t)(L >= t.r[3]);                             // code >= 4
  const uint32_t m = (t.u[5] & hi) | (t.u[1] & ~hi);
  const uint32_t mid = 0u - (uint32_t)(L >= __uint_as_float(m));               // code >= 6, or >= 2
  const uint32_t lo_hi = (t.u[6] & mid) | (t.u[4] & ~mid), lo_lo = (t.u[2] & mid) | (t.u[0] & ~mid);
  const float lo = __uint_as_float((lo_hi & hi) | (lo_lo & ~hi));
  const uint32_t mag = (hi & 4u) | (mid & 2u) | (uint32_t)(L > lo);
  return mag | ((b >> 12) & 8u);
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

// One thread per 16-element block at a time: two 16-byte loads (8 BF16 each),
// one 64-bit store of the 16 codes, one scale byte.  Each thread loads
// kQuantB blocks (blockDim apart) before it encodes any of them.
constexpr int kQuantB = 2;

struct BlockCodes {
  uint32_t lo, hi, scode;  // codes of elements 0..7 and 8..15, scale code
};

__device__ __forceinline__ uint32_t half_codes(const uint4 v, const ElemThresholds& t) {
  const uint32_t e[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                         v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= element_code(e[i], t) << (4 * i);
  return word;
}

// Largest magnitude (bits & 0x7FFF) of 8 BF16, by lane-wise 16-bit maxima.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2_t mag2(uint32_t x) { return __builtin_bit_cast(u16x2_t, x & 0x7FFF7FFFu); }

__device__ __forceinline__ uint32_t half_max(const uint4 v) {
  const u16x2_t a = __builtin_elementwise_max(__builtin_elementwise_max(mag2(v.x), mag2(v.y)),
                                              __builtin_elementwise_max(mag2(v.z), mag2(v.w)));
  return max((uint32_t)a[0], (uint32_t)a[1]);
}

__device__ __forceinline__ BlockCodes quantize_block(const uint4 v0, const uint4 v1, uint32_t amax_b, uint32_t sa,
                                                     int ea) {
  const uint32_t bam = max(half_max(v0), half_max(v1));
  const uint32_t sc = e4m3_scale_code(bam, sa, ea);   // evaluated always: a select, not a branch
  const uint32_t scode = (amax_b & 0x7FFFu) ? sc : 0u;
  const ElemThresholds t = element_thresholds(scode, sa, ea);
  return BlockCodes{half_codes(v0, t), half_codes(v1, t), scode};
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

// Over a stack, blockIdx.y picks the matrix (n_blk blocks each).  Iterations
// whose kQuantB blocks all exist run without a branch between loads, codes and
// stores, so the compiler interleaves the blocks; only the grid's last
// iteration takes the guarded path.
// FROM_TSCALE: amax_p holds the tensor scale (amax recovered from it), else amax.
template <bool DECODE, bool FROM_TSCALE = false>
__global__ void __launch_bounds__(256) quantize_kernel(const uint4* __restrict__ w, int64_t n_blk,
                                                       const float* __restrict__ amax_p,
                                                       uint2* __restrict__ packed,
                                                       uint8_t* __restrict__ scales,
                                                       uint4* __restrict__ decoded, const float* ts_w = nullptr,
                                                       float* ts_x = nullptr, float* ts_y = nullptr) {
  if constexpr (DECODE) {
    // NVFP4 x NVFP4: one thread also writes ts_x = fl32(amax / 2688) and ts_y = fl32(ts_w * ts_x).  Every
    // workgroup reads only amax_p, which is neither of them; the linear that follows reads ts_y.
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      const float tx = __fdiv_rn(amax_p[0], 2688.0f);
      ts_x[0] = tx;
      ts_y[0] = ts_w[0] * tx;
    }
  }
  w += (int64_t)blockIdx.y * 2 * n_blk;
  packed += (int64_t)blockIdx.y * n_blk;
  scales += (int64_t)blockIdx.y * n_blk;
  // amax is a BF16 value held in FP32 (or recovered from the tensor scale)
  const uint32_t amax_b = FROM_TSCALE ? amax_bits_from_tscale(amax_p[blockIdx.y])
                                      : __float_as_uint(amax_p[blockIdx.y]) >> 16;
  uint32_t sa;
  int ea;
  bf16_split(amax_b & 0x7FFFu, sa, ea);
  const int64_t B = blockDim.x;
  const int64_t stride = (int64_t)gridDim.x * B * kQuantB;
  for (int64_t b0 = (int64_t)blockIdx.x * B * kQuantB + threadIdx.x; b0 < n_blk; b0 += stride) {
    uint4 v[2 * kQuantB];
    if (b0 + (kQuantB - 1) * B < n_blk) {
#pragma unroll
      for (int u = 0; u < kQuantB; ++u) {
        v[2 * u] = w[2 * (b0 + u * B)];
        v[2 * u + 1] = w[2 * (b0 + u * B) + 1];
      }
      BlockCodes q[kQuantB];
#pragma unroll
      for (int u = 0; u < kQuantB; ++u) q[u] = quantize_block(v[2 * u], v[2 * u + 1], amax_b, sa, ea);
#pragma unroll
      for (int u = 0; u < kQuantB; ++u) store_block<DECODE>(b0 + u * B, q[u], packed, scales, decoded);
    } else {
#pragma unroll
      for (int u = 0; u < kQuantB; ++u) {
        const int64_t blk = b0 + u * B;
        if (blk < n_blk) {
          store_block<DECODE>(blk, quantize_block(w[2 * blk], w[2 * blk + 1], amax_b, sa, ea), packed, scales,
                              decoded);
        }
      }
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
  {
    const float s = e4m3_to_f32(sbyte);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t pair = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t c = (p >> (8 * j + 4 * q)) & 0xFu;
        float v = e2m1_mag_to_f32(c & 7u) * s;  // exact
        v = v * t;                              // one FP32 rounding
        if (c & 8u) v = -v;
        pair |= f32_to_bf16_rne(v) << (16 * q);
      }
      o[j] = pair;
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
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
  const unsigned nb = grid_for(n_vec, 256 * kAmaxU, kAmaxBlocks);
  amax_partial_kernel<<<dim3(nb, (unsigned)count), 256, 0, s>>>(reinterpret_cast<const uint4*>(w), n_vec, part, n_vec,
                                                                n_vec);
  amax_reduce_kernel<false><<<dim3(1, (unsigned)count), 256, 0, s>>>(part, (int)nb, amax, n_vec);
}

void launch_tscale_set_stack(const uint16_t* w, int64_t count, int64_t n_elems, uint32_t* part, float* tscale,
                             hipStream_t s) {
  const int64_t n_vec = n_elems / 8;
  const unsigned nb = grid_for(n_vec, 256 * kAmaxU, kAmaxBlocks);
  amax_partial_kernel<<<dim3(nb, (unsigned)count), 256, 0, s>>>(reinterpret_cast<const uint4*>(w), n_vec, part, n_vec,
                                                                n_vec);
  amax_reduce_kernel<true><<<dim3(1, (unsigned)count), 256, 0, s>>>(part, (int)nb, tscale, n_vec);
}

void launch_quantize_from_tscale(const uint16_t* w, int64_t count, int64_t n_elems, const float* tscale,
                                 uint8_t* packed, uint8_t* scales, hipStream_t s) {
  const int64_t n_blk = n_elems / 16;
  quantize_kernel<false, true><<<dim3(grid_for(n_blk, 256 * kQuantB, 1 << 20), (unsigned)count), 256, 0, s>>>(
      reinterpret_cast<const uint4*>(w), n_blk, tscale, reinterpret_cast<uint2*>(packed), scales, nullptr);
}

void launch_finalize_tscale(const float* amax, float* tscale, int64_t count, hipStream_t s) {
  finalize_tscale_kernel<<<(unsigned)((count + 63) / 64), 64, 0, s>>>(amax, tscale, count);
}

void launch_quantize(const uint16_t* w, int64_t count, int64_t n_elems, const float* amax, uint8_t* packed,
                     uint8_t* scales, hipStream_t s) {
  const int64_t n_blk = n_elems / 16;
  quantize_kernel<false><<<dim3(grid_for(n_blk, 256 * kQuantB, 1 << 20), (unsigned)count), 256, 0, s>>>(
      reinterpret_cast<const uint4*>(w), n_blk, amax, reinterpret_cast<uint2*>(packed), scales, nullptr);
}

void launch_quantize_decode(const uint16_t* w, int64_t n_elems, const float* amax, uint8_t* packed, uint8_t* scales,
                            uint16_t* decoded, const float* ts_w, float* ts_x, float* ts_y, hipStream_t s) {
  const int64_t n_blk = n_elems / 16;
  quantize_kernel<true><<<dim3(grid_for(n_blk, 256 * kQuantB, 1 << 20), 1u), 256, 0, s>>>(
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
