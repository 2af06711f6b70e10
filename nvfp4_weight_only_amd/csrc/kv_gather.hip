// Paged FP4 KV-cache gather to FP16 / BF16 (imp "docs/quantization.md",
// KV-cache paragraphs: an NVFP4 KV cache keeps E2M1 values with UE4M3
// micro-scales, an MXFP4 one the same nibbles with UE8M0 micro-scales per 32;
// for chunked prefill the past chunks' K/V are gathered from the paged cache
// into FP16 before attention).
//
// Cache (one per layer and per K or V): pages of block_size tokens,
//   codes  [num_blocks, block_size, heads, head_dim / 2]   (element 2j low nibble of byte j)
//   scales [num_blocks, block_size, heads, head_dim / G]   (G = 16 E4M3, or 32 UE8M0)
// plus, for NVFP4, one FP32 tensor scale.  A page's token rows are contiguous,
// and so are the output rows of consecutive tokens of one sequence, so one
// workgroup per (sequence, page of its block table) streams the page as a flat
// run of 8-element pieces: lane l of a wavefront reads code word l (4 bytes)
// and writes output piece l (16 bytes), so every store instruction covers 1 KB
// of consecutive output.  The output goes out with nontemporal stores: it is
// read by the attention that follows, not by this kernel, and streaming it past
// the caches took the gather from 3.6 to 5.75 TB/s (a plain fill of the same
// output writes 6.0 TB/s on the same GPU).
//
// Values (both sides exact up to the final rounding):
//   NVFP4  RNE_out(fl32(fl32(E2M1 * E4M3) * tscale)): the FP4 conversion at
//          scale 1.0 gives E2M1 exactly, the product with the E4M3 value has
//          at most 6 significant bits (exact in FP32), then one FP32 multiply;
//   MXFP4  RNE_out(E2M1 * 2^(e - 127)): ldexp of the exact E2M1 value (exact,
//          or infinity past FP32's range), scale byte 0xFF NaN.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {
namespace {

constexpr int kKvThreads = 256, kKvUnroll = 8;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct KvArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tscale;
  int64_t num_blocks, block_size, row_elems;  // row_elems = heads * head_dim, a multiple of 16
  const int32_t* block_table;                 // [seqs, max_blocks]
  int64_t max_blocks;
  const int32_t* seq_lens;   // [seqs]
  const int32_t* dst_start;  // [seqs]
  uint16_t* out;             // [out_rows, row_elems]
  int64_t out_rows;
};

template <bool BF16>
__device__ __forceinline__ uint32_t kv_pack2(float a, float b) {
  if constexpr (BF16) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
  } else {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    const f16x2_t r = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, r);
  }
}

// Elements 2 SEL, 2 SEL + 1 of word p, exact E2M1 values.
template <int SEL>
__device__ __forceinline__ float2 kv_e2m1x2(uint32_t p) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, SEL);
  return make_float2(v[0], v[1]);
}

// One byte of codes (2 elements) -> one output pair.
template <bool MX, bool BF16, int SEL>
__device__ __forceinline__ uint32_t kv_pair(uint32_t p, float s, float ts, int e) {
  const float2 v = kv_e2m1x2<SEL>(p);
  if constexpr (MX) {
    return kv_pack2<BF16>(e == 255 ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(v.x, e - 127),
                          e == 255 ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(v.y, e - 127));
  } else {
    return kv_pack2<BF16>((v.x * s) * ts, (v.y * s) * ts);
  }
}

// 8 elements (code word c, scale byte sb) -> one 16-byte output piece.
template <bool MX, bool BF16>
__device__ __forceinline__ u32x4_t kv_piece(uint32_t c, uint32_t sb, float ts) {
  const float s = MX ? 1.0f : e4m3_to_f32(sb);
  const int e = (int)sb;
  return u32x4_t{kv_pair<MX, BF16, 0>(c, s, ts, e), kv_pair<MX, BF16, 1>(c, s, ts, e),
                 kv_pair<MX, BF16, 2>(c, s, ts, e), kv_pair<MX, BF16, 3>(c, s, ts, e)};
}

// Workgroup (s, b): tokens b * block_size .. of sequence s, from page
// block_table[s, b].  Tokens past min(seq_lens[s], max_blocks * block_size)
// are not gathered; a page id outside [0, num_blocks) gives zero rows; output
// rows outside [0, out_rows) are skipped.  Each thread loads kKvUnroll pieces'
// codes and scales before it converts and stores any of them.
template <bool MX, bool BF16>
__global__ void __launch_bounds__(kKvThreads) kv_gather_kernel(KvArgs a) {
  const int64_t wg = blockIdx.x;
  const int64_t s = wg / a.max_blocks, b = wg - s * a.max_blocks;
  const int64_t cap = a.max_blocks * a.block_size;
  int64_t len = a.seq_lens[s];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int64_t t0 = b * a.block_size;
  if (t0 >= len) return;
  const int64_t ntok = len - t0 < a.block_size ? len - t0 : a.block_size;
  const int64_t page = a.block_table[s * a.max_blocks + b];
  const bool valid = page >= 0 && page < a.num_blocks;
  const int64_t dst0 = (int64_t)a.dst_start[s] + t0;
  const int64_t pieces = ntok * a.row_elems / 8;            // 8-element pieces to write
  const int64_t page_pieces = a.block_size * a.row_elems / 8;
  const uint32_t* cp = reinterpret_cast<const uint32_t*>(a.codes) + (valid ? page : 0) * page_pieces;
  const uint8_t* sp = a.scales + (valid ? page : 0) * page_pieces / (MX ? 4 : 2);
  u32x4_t* op = reinterpret_cast<u32x4_t*>(a.out + dst0 * a.row_elems);
  const float ts = MX ? 1.0f : *a.tscale;
  const int tid = threadIdx.x;

  for (int64_t o0 = 0; o0 < pieces; o0 += kKvThreads * kKvUnroll) {
    uint32_t c[kKvUnroll], sb[kKvUnroll];
#pragma unroll
    for (int u = 0; u < kKvUnroll; ++u) {
      int64_t o = o0 + u * kKvThreads + tid;
      o = o < page_pieces ? o : page_pieces - 1;  // the page is whole in memory
      c[u] = valid ? cp[o] : 0u;
      sb[u] = valid ? sp[MX ? o >> 2 : o >> 1] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kKvUnroll; ++u) {
      const int64_t o = o0 + u * kKvThreads + tid;
      if (o >= pieces) continue;
      const int64_t row = dst0 + (8 * o) / a.row_elems;
      if (row < 0 || row >= a.out_rows) continue;
      const u32x4_t v = valid ? kv_piece<MX, BF16>(c[u], sb[u], ts) : u32x4_t{0u, 0u, 0u, 0u};
      __builtin_nontemporal_store(v, op + o);
    }
  }
}

}  // namespace

void launch_kv_gather(bool mx, bool bf16, const uint8_t* codes, const uint8_t* scales, const float* tscale,
                      int64_t num_blocks, int64_t block_size, int64_t row_elems, const int32_t* block_table,
                      int64_t max_blocks, const int32_t* seq_lens, const int32_t* dst_start, int64_t seqs,
                      uint16_t* out, int64_t out_rows, hipStream_t s) {
  const KvArgs a{codes, scales, tscale, num_blocks, block_size, row_elems, block_table, max_blocks,
                 seq_lens, dst_start, out, out_rows};
  const dim3 grid((unsigned)(seqs * max_blocks));
  if (mx) {
    if (bf16) kv_gather_kernel<true, true><<<grid, kKvThreads, 0, s>>>(a);
    else kv_gather_kernel<true, false><<<grid, kKvThreads, 0, s>>>(a);
  } else {
    if (bf16) kv_gather_kernel<false, true><<<grid, kKvThreads, 0, s>>>(a);
    else kv_gather_kernel<false, false><<<grid, kKvThreads, 0, s>>>(a);
  }
}

}  // namespace nvfp4
