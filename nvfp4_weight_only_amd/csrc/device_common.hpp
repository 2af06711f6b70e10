// Device helpers for the gfx950 NVFP4 kernels: number formats and packing.
//
// Formats (homepage "Raphael Friedmann", NVFP4 bit diagram; imp
// "docs/quantization.md", imp-quantize section and the micro-scale paragraph):
//   E2M1 nibble  s|e1 e0|m, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7),
//                code 8..15 the negatives (8 = -0);
//   E4M3 byte    OCP E4M3FN: s|eeee|mmm, bias 7, e = 0 subnormal m/8 * 2^-6,
//                0x7F/0xFF NaN, max 448;
//   packing      element 2j in the low nibble of byte j, 2j+1 in the high nibble;
//                one E4M3 scale per 16 consecutive K elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Scalars.
// ---------------------------------------------------------------------------

// E4M3FN byte -> float, exact (branch-free for the non-negative codes used as scales).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  const float vn = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  const float vs = (float)m * 0x1p-9f;                               // m/8 * 2^-6
  float v = e ? vn : vs;
  if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
  return (c & 0x80u) ? -v : v;
}

// E2M1 magnitude code 0..7 -> float, exact.
__device__ __forceinline__ float e2m1_mag_to_f32(uint32_t mag) {
  const uint32_t e = (mag >> 1) & 3u, m = mag & 1u;
  const uint32_t nb = ((e + 126u) << 23) | (m << 22);   // 2^(e-1) * (1 + m/2)
  return __uint_as_float(e ? nb : (m ? 0x3F000000u : 0u));
}

// float -> BF16 bits, round to nearest even (NaN -> canonical quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// BF16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// ---------------------------------------------------------------------------
// Eight packed elements (one 32-bit word) -> BF16.
// ---------------------------------------------------------------------------

// BF16 bit patterns of the E2M1 magnitudes, split into byte planes for v_perm_b32.
// magnitude:       0     0.5   1     1.5   2     3     4     6
// low byte:        00    00    80    C0    00    40    80    C0
// high byte:       00    3F    3F    3F    40    40    40    40
constexpr uint32_t kLoLut0 = 0xC0800000u;  // magnitudes 0..3
constexpr uint32_t kLoLut1 = 0xC0804000u;  // magnitudes 4..7
constexpr uint32_t kHiLut0 = 0x3F3F3F00u;
constexpr uint32_t kHiLut1 = 0x40404040u;

// Unscaled decode of the 8 elements of `p` into 4 BF16 pairs in the order
//   out.x = (e0, e2), out.y = (e4, e6), out.z = (e1, e3), out.w = (e5, e7)
// (low half first).  Pair the result with activations permuted the same way.
// Byte-permute lookups: 2 selector ops, 4 table lookups, 3 sign ops, 4 interleaves.
__device__ __forceinline__ uint4 e2m1x8_to_bf16_interleaved(uint32_t p) {
  const uint32_t se = p & 0x07070707u;          // magnitudes of elements 0, 2, 4, 6
  const uint32_t so = (p >> 4) & 0x07070707u;   // magnitudes of elements 1, 3, 5, 7
  const uint32_t lo_e = __builtin_amdgcn_perm(kLoLut1, kLoLut0, se);
  const uint32_t hi_e = __builtin_amdgcn_perm(kHiLut1, kHiLut0, se) | ((p << 4) & 0x80808080u);
  const uint32_t lo_o = __builtin_amdgcn_perm(kLoLut1, kLoLut0, so);
  const uint32_t hi_o = __builtin_amdgcn_perm(kHiLut1, kHiLut0, so) | (p & 0x80808080u);
  uint4 r;
  r.x = __builtin_amdgcn_perm(hi_e, lo_e, 0x05010400u);
  r.y = __builtin_amdgcn_perm(hi_e, lo_e, 0x07030602u);
  r.z = __builtin_amdgcn_perm(hi_o, lo_o, 0x05010400u);
  r.w = __builtin_amdgcn_perm(hi_o, lo_o, 0x07030602u);
  return r;
}

// Permute 8 BF16 activations (4 natural-order pairs) into the order used above.
__device__ __forceinline__ uint4 bf16x8_interleave(uint4 d) {
  uint4 r;
  r.x = __builtin_amdgcn_perm(d.y, d.x, 0x05040100u);  // (x0, x2)
  r.y = __builtin_amdgcn_perm(d.w, d.z, 0x05040100u);  // (x4, x6)
  r.z = __builtin_amdgcn_perm(d.y, d.x, 0x07060302u);  // (x1, x3)
  r.w = __builtin_amdgcn_perm(d.w, d.z, 0x07060302u);  // (x5, x7)
  return r;
}

// Scaled decode: 8 elements of `p` times the block scale `s` (an E4M3 value)
// as BF16 pairs in natural order.  E2M1 * E4M3 has at most 6 significant bits
// and lies in [2^-10, 2688], so the product is exact in FP32 and its top half
// is the exact BF16 value.
__device__ __forceinline__ uint4 e2m1x8_scaled_to_bf16(uint32_t p, float s) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t c0 = (p >> (8 * j)) & 0xFu, c1 = (p >> (8 * j + 4)) & 0xFu;
    const uint32_t b0 = (__float_as_uint(e2m1_mag_to_f32(c0 & 7u) * s) >> 16) | ((c0 & 8u) << 12);
    const uint32_t b1 = (__float_as_uint(e2m1_mag_to_f32(c1 & 7u) * s) >> 16) | ((c1 & 8u) << 12);
    o[j] = b0 | (b1 << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Unscaled decode with the gfx950 conversion instruction: byte `SEL` of `p`
// (elements 2*SEL, 2*SEL+1) -> one BF16 pair in natural order.  The
// instruction multiplies by 2^exponent(scale) only, so a scale of 1.0 gives the
// exact E2M1 values (including -0 for code 8).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16(uint32_t p) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p, 1.0f, SEL));
}

// Scaled decode with the conversion instruction: byte SEL of `p` (elements
// 2*SEL, 2*SEL+1) times the E4M3 block scale `s`, as one BF16 pair in natural
// order.  The FP4 -> FP32 conversion at scale 1.0 gives the exact E2M1 values;
// E2M1 * E4M3 has at most 6 significant bits, so the FP32 products are exact
// and their high halves are the exact BF16 values (signs and -0 included).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_scaled_to_bf16(uint32_t p, float s) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, SEL);
  return __builtin_amdgcn_perm(__float_as_uint(v[1] * s), __float_as_uint(v[0] * s), 0x07060302u);
}

// Dequantized BF16 pair: byte SEL of `p` (elements 2*SEL, 2*SEL+1) as
// RNE_bf16(fl32(fl32(E2M1 * s) * t)).  E2M1 from the conversion instruction
// (exact, -0 kept), E2M1 * s exact, one FP32 rounding by t, then the
// nearest-even BF16 conversion (v_cvt_pk_bf16_f32).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_dequant_bf16(uint32_t p, float s, float t) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, SEL);
  const f32x2_t a = {(v[0] * s) * t, (v[1] * s) * t};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2v_t));
}

// Eight elements (one packed word) dequantized to BF16 with block scale s and
// tensor scale t (finite): four natural-order pairs.  A NaN scale (E4M3 0x7F /
// 0xFF) gives the canonical quiet NaN 0x7FC0 in every element.
__device__ __forceinline__ uint4 e2m1x8_dequant_bf16(uint32_t p, float s, float t) {
  const uint4 r = make_uint4(e2m1x2_dequant_bf16<0>(p, s, t), e2m1x2_dequant_bf16<1>(p, s, t),
                             e2m1x2_dequant_bf16<2>(p, s, t), e2m1x2_dequant_bf16<3>(p, s, t));
  return s == s ? r : make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
}

// Eight elements of `p` times `s` as four natural-order BF16 pairs.
__device__ __forceinline__ uint4 e2m1x8_scaled_to_bf16_hw(uint32_t p, float s) {
  return make_uint4(e2m1x2_scaled_to_bf16<0>(p, s), e2m1x2_scaled_to_bf16<1>(p, s), e2m1x2_scaled_to_bf16<2>(p, s),
                    e2m1x2_scaled_to_bf16<3>(p, s));
}

// Two E4M3 (OCP E4M3FN) bytes -> two floats with the gfx950 FP8 conversion:
// bytes 0 and 1 of `v` when HI is false, bytes 2 and 3 when HI is true.
template <bool HI>
__device__ __forceinline__ float2 e4m3x2_to_f32(uint32_t v) {
  const auto r = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, HI);
  return make_float2(r[0], r[1]);
}

// ---------------------------------------------------------------------------
// Streaming loads: data read once per call (weights and their scales) carry
// the nontemporal hint, so that they do not displace what is
// reused from L2.  On a 100 MB read this took a plain 16-byte-per-lane read
// from 17.9 to 16.0 us.  It pays only where each load instruction reads whole
// lines: with half lines per instruction (the line's other half read by the
// next one) or 4- and 1-byte lanes, the lines are dropped before their second
// use and the kernels slowed by 5-30 %.
// ---------------------------------------------------------------------------
typedef uint32_t stream_u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const stream_u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const stream_u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t ld_stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// ---------------------------------------------------------------------------
// Dot products and wave reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Lanes of one wavefront exchanging data through LDS: the stores before this
// point are visible to every lane's loads after it.  Without it the exchange
// is a data race in HIP's memory model, and the compiler may legally move a
// lane's load of another lane's slot above that lane's store (per thread, the
// two addresses differ).  Costs no instruction at wavefront scope.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Partial sums of a split-K exchange, four consecutive output rows n0 .. n0 + 3
// (n0 a multiple of 4) of one activation row; row points at that activation
// row's partial sums (a multiple of 16 values long).  Inside the aligned
// 16-row span s = n0 & ~15, the 4-row group j = (n0 / 4) % 4 keeps its values
// 0 and 1 at s + 2 j and values 2 and 3 at s + 8 + 2 j, so the four groups of
// a span, stored by one instruction, fill whole 32-byte sectors (in row order
// each instruction's 4-byte pieces would lie 16 bytes apart).  Device-scope
// relaxed atomic stores and loads of 8 bytes: written through to the device's
// coherence point, so the release that follows finds no dirty L2 lines of
// them to write back.
__device__ __forceinline__ void splitk_store_rows4(float* row, int64_t n0, f32x4_t v) {
  float* p = row + (n0 & ~(int64_t)15) + 2 * ((n0 >> 2) & 3);
  const uint64_t lo = (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32);
  const uint64_t hi = (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p + 8), hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4_t splitk_load_rows4(const float* row, int64_t n0) {
  const float* p = row + (n0 & ~(int64_t)15) + 2 * ((n0 >> 2) & 3);
  const uint64_t lo = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi =
      __hip_atomic_load(reinterpret_cast<const uint64_t*>(p + 8), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4_t{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)), __uint_as_float((uint32_t)hi),
                 __uint_as_float((uint32_t)(hi >> 32))};
}

// ---------------------------------------------------------------------------
// Split-K hand-off between the workgroups that share one block of outputs,
// each having stored its FP32 partial sums (splitk_store_rows4).  In HIP's
// memory model: the first barrier orders every thread's stores before thread
// 0's release read-modify-write of the block's arrival counter (device
// scope); the workgroup whose increment completes the count performs a
// device-scope acquire fence, and the second barrier orders that before its
// threads' loads of the other slices' sums, so those loads see the stores
// (release sequence on the counter, then barrier transitivity).  On
// gfx950 the release writes back the XCD's L2 and the acquire invalidates the
// CU's L1 and the XCD's L2 lines from other agents, because the eight XCDs'
// L2s are not coherent with each other; only the last workgroup of a block
// pays for the invalidation.  The explicit vmcnt(0) before the first barrier
// also makes every thread's stores complete to L2 before thread 0 releases.
// Returns true in every thread of the last workgroup, which also resets the
// counter to zero for the next launch (the launch boundary orders that).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool splitk_arrive(uint32_t* count, int slices) {
  __shared__ int last_flag;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == (uint32_t)(slices - 1);
    if (last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    last_flag = last;
  }
  __syncthreads();
  return last_flag != 0;
}

}  // namespace nvfp4
