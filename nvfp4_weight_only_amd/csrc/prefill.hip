// Prefill W4A16 GEMM for K a multiple of 256 on gfx950: Y = X W^T with bf16
// v_mfma_f32_32x32x16_bf16 and FP32 accumulation (model card
// "Qwen3.8-27B-NVFP4 (compressed-tensors)": weights NVFP4, activations BF16;
// imp "docs/quantization.md", NVFP4 kernel pipeline: prefill is the dense GEMM).
//
// A workgroup computes a 128 x 272 tile of Y (272 = 17 x 16 divides the MLP
// width 17408 into 64 tiles: 256 workgroups at m = 512) with four wavefronts,
// one per SIMD.  LDS read bandwidth (about 64 B per clock per CU for 128-bit
// reads) is what bounds a GEMM that dequantizes through LDS, so:
//   * every wavefront owns 64 of the 272 columns for all 128 rows: the BF16
//     activations are read from LDS by every wavefront, but each weight element
//     is read (packed, 4 bits) and decoded by exactly one wavefront, straight
//     into the MFMA B operand;
//   * columns 256..271 form a fifth 32-column MFMA tile (upper 16 columns
//     unused) whose four 16-wide K steps per 64-column step are shared out one
//     per wavefront; its partial sums are added in wavefront order at the end;
//   * activations (128 rows x 64 K per step, a 5-stage ring), packed weights
//     and scales (272 rows x 256 K per group, double-buffered) move from global
//     memory to LDS with global_load_lds_dwordx4, whole 128-byte lines per
//     instruction, without passing through registers.
//
// K order inside a 64-element step: lane half h (lanes 32h .. 32h + 31) of an
// MFMA covers the step's elements [32h, 32h + 32); K step s (0..3) takes
// [32h + 8s, 32h + 8s + 8).  A weight lane thus reads 16 contiguous packed bytes
// per step; activations follow the same order (a dot product does not depend on
// the order of its terms; only the FP32 summation order changes).
#include <utility>

#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) const void pd_lds_t;

constexpr int kPdBM = 128, kPdBN = 272, kPdBK = 64, kPdGroupK = 256;

struct PdArgs {
  const uint16_t* x;  // [m, k]
  int64_t m, n, k;
  const uint8_t* packed;
  const uint8_t* scales;
  const float* tscale;
  uint16_t* y;
  int n_tiles, m_tiles;
  // Grouped form (an expert stack): the routed pairs sorted by expert, as
  // built by the grouping kernels (see PdGroups), and the stack's layout.
  const int32_t* groups;
  int64_t topk, experts, w_stride;  // w_stride: packed bytes per expert
  // Split K for the tiles past the last whole round (plain form only): the
  // first sk_dp tiles run one per workgroup over the whole K (the whole grid
  // when sk_tail = 0); each of the remaining sk_tail tiles is split into sk_c
  // slices of whole 256-element groups, one workgroup each, launched after
  // the whole tiles.  A split tile's workgroups exchange FP32 partial tiles in
  // `part` (sk_c slots per tile) and meet at its arrival counter in `count`
  // (see pd_exchange).
  int sk_dp, sk_tail, sk_c;
  float* part;
  uint32_t* count;
};


// FP32 partial tile of one (tile, slice): per wavefront 34 float4 per lane
// (its 8 accumulator tiles of 16 items, then the fifth tile's 8 items).
constexpr int kPdPartVec = 34;
constexpr int64_t kPdPartBytes = 4 * kPdPartVec * 64 * 16;  // 139,264 = 128 x 272 x 4

// Layout of the grouping workspace (int32): cnt[E] (the sort's counters),
// pair_off[E + 1] (first sorted position of each expert's pairs; pair_off[E]
// = V, the pairs with a valid expert id), tile_off[E + 1] (first 128-row tile
// of each expert), perm[pairs] (pair indices grouped by expert, then the V..
// pairs - 1 invalid ones).
struct PdGroups {
  const int32_t* pair_off;
  const int32_t* tile_off;
  const int32_t* perm;
};

__device__ __forceinline__ PdGroups pd_groups(const PdArgs& p) {
  const int32_t* g = p.groups;
  return PdGroups{g + p.experts, g + 2 * p.experts + 1, g + 3 * p.experts + 2};
}

// LDS (16-byte slots):
//   x stage: activation row r (of 128), piece p (8 elements) at 8 r + (p ^ (r & 7))
//            (the XOR makes 8 consecutive rows at the same piece hit different banks);
//   w group: weight row r (of 272) in 9 slots at 9 r: its 8 packed pieces of 32
//            elements, then its 16 scale bytes.  The odd row stride spreads 16
//            consecutive rows over all banks, and a scale byte travels with
//            its row's weights instead of in a 64-row gather of its own.
constexpr int kPdWSlots = 9;
struct PdX {
  uint4 v[kPdBM * 8];
};
struct PdW {
  uint4 v[kPdBN * kPdWSlots];
};
// Five activation stages (16 KB each) and two weight groups (38.25 KB):
// 160,256 bytes of the 160 KB of LDS.
constexpr int kPdXStages = 5;
struct PdLds {
  PdX xs[kPdXStages];
  PdW wg[2];
  int32_t rowmap[kPdBM];  // grouped form: the output row (pair index) of each tile row
};

// One global_load_lds_dwordx4 from a per-lane 64-bit address (the weight group
// loads mix the packed and the scale arrays in one instruction).
__device__ __forceinline__ void pd_lds_dma16_ptr(const void* src, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// One global_load_lds_dwordx4: 16 bytes per lane from base + off (a
// wavefront-uniform base and a per-lane 32-bit byte offset) to LDS address
// lds + 16 * lane.  Written out rather than through the compiler builtin, whose
// wait insertion loses track of which buffer a pending load writes at a loop
// head and drains every load in flight; the instruction has no register
// result, and the kernel orders LDS reads after it with explicit vmcnt waits.
// M0 is declared clobbered, so the compiler keeps nothing of its own there.
__device__ __forceinline__ void pd_lds_dma16(const void* base, uint32_t off, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  const uint64_t b = (uint64_t)(uintptr_t)base;
  // readfirstlane returns int: widen through uint32_t, never by sign extension.
  const uint64_t bs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(bs), "{m0}"(m0) : "memory");
}

template <typename U>
__device__ __forceinline__ uint32_t pd_lds_addr(const U* p) {
  return (uint32_t)(uintptr_t)(pd_lds_t*)p;
}

template <int N>
__device__ __forceinline__ void pd_wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// vmcnt(N) and lgkmcnt(0) in one wait.  Before a step's barrier the LDS reads
// of the previous step have long completed; saying so lets the MFMAs that use
// them start without waiting behind the reads issued after the barrier (the
// LDS counter tracks at most 15 reads in flight).
template <int N>
__device__ __forceinline__ void pd_wait_vmcnt_lds0() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// Load instructions per wavefront: X 4 per step (16 instructions of 8 rows);
// weights and scales 10 per group (272 x 9 slots = 38.25 instructions of 64
// slots; the last instruction is placed to end at slot 2448, and the spare
// repeats it).
constexpr int kPdLX = 4, kPdLW = 10;
constexpr int kPdWLast = kPdBN * kPdWSlots - 64;  // first slot of the last weight instruction

// Per-lane sources of the loads: activation byte offsets from the tile's first
// row at K = 0, and the group 0 addresses of the weight / scale slots, with a
// bit per instruction that marks a scale slot (16 bytes further per group
// instead of 128).
struct PdSrc {
  uint32_t x[kPdLX];
  const uint8_t* w[kPdLW];
  uint32_t wscale;
};

// The loads of one step: the activation base, the weight group index, and LDS
// byte addresses of the destination buffers.
struct PdDma {
  const uint8_t* xb;
  int64_t gc;
  uint32_t xs, wg;
};

// Bases of the loads of step t into X stage `xst` and, when the step starts a
// group, of group t / 4 into weight / scale buffer (t / 4) % 2.  Past the
// end, the last step / group is loaded again into buffers nothing reads.
__device__ __forceinline__ PdDma pd_dma_begin(const PdArgs& p, int64_t m0, int64_t n0, int t, int nsteps,
                                              const PdLds& L, int xst) {
  const int tc = t < nsteps ? t : nsteps - 1;
  const int64_t gc = tc >> 2;
  const int gb = (t >> 2) & 1;
  (void)n0;
  return PdDma{reinterpret_cast<const uint8_t*>(p.x + m0 * p.k) + (int64_t)tc * (2 * kPdBK), gc,
               pd_lds_addr(&L.xs[xst]), pd_lds_addr(&L.wg[gb])};
}

// Load instruction I of a step (place in group P): 0..3 activations, then at a
// group start 4..13 weight rows with their scales; nothing for other I.
template <int P, int I>
__device__ __forceinline__ void pd_dma_one(const PdSrc& src, const PdDma& d, int w) {
  if constexpr (I < kPdLX) {
    pd_lds_dma16(d.xb, src.x[I], d.xs + 1024 * (w + 4 * I));
  } else if constexpr (P == 0 && I < kPdLX + kPdLW) {
    constexpr int i = I - kPdLX;
    const int q0 = 64 * (w + 4 * i);
    const int q = q0 < kPdWLast ? q0 : kPdWLast;
    const int64_t step = (src.wscale >> i) & 1u ? kPdGroupK / 16 : kPdGroupK / 2;
    pd_lds_dma16_ptr(src.w[i] + d.gc * step, d.wg + 16 * q);
  }
}

template <int P, int... I>
__device__ __forceinline__ void pd_dma_all(const PdSrc& src, const PdDma& d, int w, std::integer_sequence<int, I...>) {
  (pd_dma_one<P, I>(src, d, w), ...);
}

// All loads of step t (before the loop).
template <int P>
__device__ __forceinline__ void pd_issue(const PdArgs& p, const PdSrc& src, int64_t m0, int64_t n0, int t, int nsteps,
                                         const PdLds& L, int xst, int w) {
  pd_dma_all<P>(src, pd_dma_begin(p, m0, n0, t, nsteps, L, xst), w,
                std::make_integer_sequence<int, kPdLX + kPdLW>{});
}

// One step's operands for one wavefront, read from LDS a step ahead of use.
struct PdFrag {
  uint4 xa[4][4];  // A fragments: row tile rt, K step s
  uint4 wb[2];     // own weight columns 64 W + 32 c + l32: 16 packed bytes (32 elements)
  uint32_t sb[2];  // their scale word for this step (bytes 4P .. 4P + 3 of the group row)
  uint32_t w5, s5;  // fifth tile: packed word of K step W and the scale word
};

// Reads of step t's operands (its place in the group is P), in two kinds:
// weights and scales from group buffer `gb`, and one K step's A fragments from
// X stage `xst`.  K order: lane half h covers the step's elements [32h, 32h + 32),
// K step s takes [32h + 8s, 32h + 8s + 8) (a dot product does not depend on the
// order of its terms; only the FP32 summation order changes).  Only plain
// reads here: anything computed from them would wait for them.
template <int P, int W>
__device__ __forceinline__ void pd_load_w(const PdLds& L, int gb, int lane, PdFrag& F) {
  const int l32 = lane & 31, h = lane >> 5;
  const PdW& Wg = L.wg[gb];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int n = 64 * W + 32 * c + l32;
    F.wb[c] = Wg.v[n * kPdWSlots + 2 * P + h];
    F.sb[c] = reinterpret_cast<const uint32_t*>(&Wg.v[n * kPdWSlots + 8])[P];
  }
  // Fifth tile rows 256 + l32 (the upper 16 lanes' rows do not exist and are clamped).
  const int n5 = 256 + (l32 < 16 ? l32 : 15);
  F.w5 = reinterpret_cast<const uint32_t*>(&Wg.v[n5 * kPdWSlots + 2 * P + h])[W];
  F.s5 = reinterpret_cast<const uint32_t*>(&Wg.v[n5 * kPdWSlots + 8])[P];
}

template <int S>
__device__ __forceinline__ void pd_load_x(const PdLds& L, int xst, int lane, PdFrag& F) {
  const int l32 = lane & 31, h = lane >> 5;
  const PdX& X = L.xs[xst];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int r = 32 * rt + l32;
    F.xa[rt][S] = X.v[r * 8 + ((4 * h + S) ^ (r & 7))];
  }
}

// Decoded B fragments: two own column tiles, four BF16 pairs each.
struct PdB {
  uint32_t v[2][4];
};

// The E4M3 scale of K step S of tile c, as a float (lane half h: blocks
// 4P + 2h and 4P + 2h + 1 of the group row; K step S uses block 4P + 2h + S / 2).
template <int S>
__device__ __forceinline__ float pd_scale(const PdFrag& F, int h, int c) {
  return e4m3x2_to_f32<false>((F.sb[c] >> (16 * h + 8 * (S >> 1))) & 0xFFu).x;
}

template <int S>
__device__ __forceinline__ uint32_t pd_word(const PdFrag& F, int c) {
  return S == 0 ? F.wb[c].x : S == 1 ? F.wb[c].y : S == 2 ? F.wb[c].z : F.wb[c].w;
}

// One MFMA with the decoded weights as the A operand and the activations as
// B: the accumulator holds the tile transposed (Y^T = W X^T), so that each
// lane ends up with 4 consecutive columns of one row of Y.
__device__ __forceinline__ void pd_mfma(f32x16_t& acc, const uint4& a, const uint32_t (&b)[4]) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, make_uint4(b[0], b[1], b[2], b[3])),
                                                __builtin_bit_cast(bf16x8_t, a), acc, 0, 0, 0);
}

// Pair J of an 8-element decode (4 instructions).
template <int J>
__device__ __forceinline__ uint32_t pd_dec(uint32_t word, float sc) {
  return e2m1x2_scaled_to_bf16<J>(word, sc);
}

// One K step S of the current step: its 8 MFMAs (row tile i / 2, column tile
// i % 2) on the decoded fragments `bc`, each followed by one pair of the next
// K step's decode into `bn` (tile i / 4), one of the step's global-to-LDS
// loads (step place P, load 8 S + i) and, for the first four, the read of one
// A fragment of the next step (K step S).  The fixed order keeps the
// decode in the MFMAs' shadow and at most a few LDS reads in flight.
template <int S, int P>
__device__ __forceinline__ void pd_kstep(const PdLds& L, int xst, int lane, const PdFrag& C, PdFrag& N,
                                         const PdB& bc, PdB& bn, f32x16_t (&acc)[4][2], const PdSrc& src,
                                         const PdDma& dma, int w) {
  const int l32 = lane & 31, h = lane >> 5;
  const PdX& X = L.xs[xst];
  const float sc0 = pd_scale<S + 1>(C, h, 0), sc1 = pd_scale<S + 1>(C, h, 1);
  const uint32_t w0 = pd_word<S + 1>(C, 0), w1 = pd_word<S + 1>(C, 1);
#define PD_G(I, DEC)                                                               \
  pd_mfma(acc[(I) / 2][(I) % 2], C.xa[(I) / 2][S], bc.v[(I) % 2]);                  \
  DEC;                                                                             \
  pd_dma_one<P, 8 * S + (I)>(src, dma, w);                                         \
  if ((I) < 4) {                                                                   \
    const int r = 32 * (I) + l32;                                                  \
    N.xa[(I) & 3][S] = X.v[r * 8 + ((4 * h + S) ^ (r & 7))];                       \
  }                                                                                \
  __builtin_amdgcn_sched_barrier(0);
  PD_G(0, bn.v[0][0] = pd_dec<0>(w0, sc0))
  PD_G(1, bn.v[0][1] = pd_dec<1>(w0, sc0))
  PD_G(2, bn.v[0][2] = pd_dec<2>(w0, sc0))
  PD_G(3, bn.v[0][3] = pd_dec<3>(w0, sc0))
  PD_G(4, bn.v[1][0] = pd_dec<0>(w1, sc1))
  PD_G(5, bn.v[1][1] = pd_dec<1>(w1, sc1))
  PD_G(6, bn.v[1][2] = pd_dec<2>(w1, sc1))
  PD_G(7, bn.v[1][3] = pd_dec<3>(w1, sc1))
#undef PD_G
}

// The decode of K step 0 of a step's operands (before the loop).
__device__ __forceinline__ void pd_decode0(const PdFrag& F, int h, PdB& b) {
  const float sc0 = pd_scale<0>(F, h, 0), sc1 = pd_scale<0>(F, h, 1);
  b.v[0][0] = pd_dec<0>(F.wb[0].x, sc0);
  b.v[0][1] = pd_dec<1>(F.wb[0].x, sc0);
  b.v[0][2] = pd_dec<2>(F.wb[0].x, sc0);
  b.v[0][3] = pd_dec<3>(F.wb[0].x, sc0);
  b.v[1][0] = pd_dec<0>(F.wb[1].x, sc1);
  b.v[1][1] = pd_dec<1>(F.wb[1].x, sc1);
  b.v[1][2] = pd_dec<2>(F.wb[1].x, sc1);
  b.v[1][3] = pd_dec<3>(F.wb[1].x, sc1);
}

// The MFMAs of one step on operands `C` (read during the previous step; `b`
// holds their K step 0 decoded) while reading the next step's operands `N`
// (X stage `xst`, group buffer `gb`, place in group PN), issuing the loads
// `dma` of the step four ahead, and decoding ahead: K steps 1..3 during the
// K step before, the fifth tile's fragment and N's K step 0 (left in `b`)
// during K step 3 and the fifth tile's MFMAs.
template <int PN, int W>
__device__ __forceinline__ void pd_step(const PdLds& L, int xst, int gb, int lane, const PdFrag& C, PdFrag& N,
                                        PdB& b, f32x16_t (&acc)[4][2], f32x16_t (&acc5)[4], const PdSrc& src,
                                        const PdDma& dma) {
  constexpr int P = (PN + 3) & 3;  // place in group of this step (and of the step it loads)
  const int l32 = lane & 31, h = lane >> 5;
  PdB t;
  pd_load_w<PN, W>(L, gb, lane, N);
  __builtin_amdgcn_sched_barrier(0);
  pd_kstep<0, P>(L, xst, lane, C, N, b, t, acc, src, dma, W);
  pd_kstep<1, P>(L, xst, lane, C, N, t, b, acc, src, dma, W);
  pd_kstep<2, P>(L, xst, lane, C, N, b, t, acc, src, dma, W);
  // K step 3: MFMAs on t; decode the fifth tile's fragment and N's K step 0, tile 0.
  const PdX& X = L.xs[xst];
  const float s5 = e4m3x2_to_f32<false>((C.s5 >> (16 * h + 8 * (W >> 1))) & 0xFFu).x;
  uint32_t b5[4];
#define PD_G3(I, DEC)                                                              \
  pd_mfma(acc[(I) / 2][(I) % 2], C.xa[(I) / 2][3], t.v[(I) % 2]);                   \
  DEC;                                                                             \
  if ((I) < 4) {                                                                   \
    const int r = 32 * (I) + l32;                                                  \
    N.xa[(I) & 3][3] = X.v[r * 8 + ((4 * h + 3) ^ (r & 7))];                       \
  }                                                                                \
  __builtin_amdgcn_sched_barrier(0);
  PD_G3(0, b5[0] = pd_dec<0>(C.w5, s5))
  PD_G3(1, b5[1] = pd_dec<1>(C.w5, s5))
  PD_G3(2, b5[2] = pd_dec<2>(C.w5, s5))
  PD_G3(3, b5[3] = pd_dec<3>(C.w5, s5))
  const float n0s = pd_scale<0>(N, h, 0), n1s = pd_scale<0>(N, h, 1);
  PD_G3(4, b.v[0][0] = pd_dec<0>(N.wb[0].x, n0s))
  PD_G3(5, b.v[0][1] = pd_dec<1>(N.wb[0].x, n0s))
  PD_G3(6, b.v[0][2] = pd_dec<2>(N.wb[0].x, n0s))
  PD_G3(7, b.v[0][3] = pd_dec<3>(N.wb[0].x, n0s))
#undef PD_G3
  // Fifth tile: K step W of rows 32 rt .. 32 rt + 31.
#define PD_G5(RT, DEC)                                \
  pd_mfma(acc5[RT], C.xa[RT][W], b5);                 \
  DEC;                                                \
  __builtin_amdgcn_sched_barrier(0);
  PD_G5(0, b.v[1][0] = pd_dec<0>(N.wb[1].x, n1s))
  PD_G5(1, b.v[1][1] = pd_dec<1>(N.wb[1].x, n1s))
  PD_G5(2, b.v[1][2] = pd_dec<2>(N.wb[1].x, n1s))
  PD_G5(3, b.v[1][3] = pd_dec<3>(N.wb[1].x, n1s))
#undef PD_G5
}

__device__ __forceinline__ int pd_next_stage(int s) { return s == kPdXStages - 1 ? 0 : s + 1; }

// Two floats as a BF16 pair, round to nearest even (v_cvt_pk_bf16_f32; a NaN
// comes out as a quiet NaN).
__device__ __forceinline__ uint32_t pd_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// Items V .. V + 3 of an accumulator times the tensor scale, as 4 BF16.
__device__ __forceinline__ uint2 pd_pack4(const f32x16_t& a, int V, float ts) {
  return make_uint2(pd_bf16x2(a[V] * ts, a[V + 1] * ts), pd_bf16x2(a[V + 2] * ts, a[V + 3] * ts));
}

// Copy the BF16 tile (128 x 272, row-major in LDS) to Y rows m0.., columns
// n0..: 34 pieces of 8 columns per row, 17 per thread.  Pieces that are whole,
// inside Y and 16-byte aligned go as one store; the others element by element.
template <bool G>
__device__ __forceinline__ void pd_store_tile(const PdArgs& p, const uint16_t* yt, int64_t m0, int64_t n0, int tid,
                                              const int32_t* rowmap) {
  const int64_t rows = p.m - m0 < kPdBM ? p.m - m0 : kPdBM;
  const int64_t cols = p.n - n0 < kPdBN ? p.n - n0 : kPdBN;
  constexpr int kPieces = kPdBN / 8;
#pragma unroll 1
  for (int j = tid; j < kPdBM * kPieces; j += 256) {
    const int r = j / kPieces, c8 = 8 * (j - r * kPieces);
    if (r >= rows || c8 >= cols) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(yt + r * kPdBN + c8);
    uint16_t* dst = p.y + (G ? (int64_t)rowmap[r] : m0 + r) * p.n + n0 + c8;
    if (c8 + 8 <= cols && ((uintptr_t)dst & 15) == 0) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
      for (int i = 0; i < 8 && c8 + i < cols; ++i) dst[i] = e[i];
    }
  }
}

// Split-K exchange of one wavefront's sums (its accumulators and its row
// tile of the fifth column tile, already summed over the wavefronts) for split
// tile xtile, shared by cnt workgroups of which this is slice sl: the partial
// tile goes to slot sl of the workspace, the tile's workgroups meet at its
// arrival counter (splitk_arrive: release / acquire at device scope), and the
// last one replaces its sums by the sum over all slices in slice order (the
// same bits whichever workgroup arrives last).  Returns false in the others,
// which are done.
template <int W>
__device__ __forceinline__ bool pd_exchange(const PdArgs& p, f32x16_t (&acc)[4][2], float4& t5a, float4& t5b, int xtile,
                                            int sl, int cnt, int lane) {
  auto slot = [&](int s, int j) {
    return p.part + ((((int64_t)xtile * p.sk_c + s) * 4 + W) * kPdPartVec + j) * 256 + 4 * lane;
  };
  auto get = [&](int j) -> f32x4_t {
    if (j < 32) {
      const f32x16_t& a = acc[j >> 3][(j >> 2) & 1];
      const int q = 4 * (j & 3);
      return f32x4_t{a[q], a[q + 1], a[q + 2], a[q + 3]};
    }
    const float4 t = j == 32 ? t5a : t5b;
    return f32x4_t{t.x, t.y, t.z, t.w};
  };
  auto put = [&](int j, f32x4_t v) {
    if (j < 32) {
      f32x16_t& a = acc[j >> 3][(j >> 2) & 1];
      const int q = 4 * (j & 3);
      a[q] = v[0]; a[q + 1] = v[1]; a[q + 2] = v[2]; a[q + 3] = v[3];
    } else if (j == 32) {
      t5a = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      t5b = make_float4(v[0], v[1], v[2], v[3]);
    }
  };
  // Ordinary 16-byte stores and loads (whole kilobytes per instruction): the
  // release of splitk_arrive writes the partial tile back from L2, the
  // acquire makes the last workgroup read it from memory.
#pragma unroll
  for (int j = 0; j < kPdPartVec; ++j) *reinterpret_cast<f32x4_t*>(slot(sl, j)) = get(j);
  if (!splitk_arrive(p.count + xtile, cnt)) return false;
  // Two halves of 17 vectors: each half's loads of every other slice are in
  // flight together.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4_t sum[17];
#pragma unroll
    for (int i = 0; i < 17; ++i) sum[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < cnt; ++s) {
#pragma unroll
      for (int i = 0; i < 17; ++i)
        sum[i] += s == sl ? get(17 * h + i) : *reinterpret_cast<const f32x4_t*>(slot(s, 17 * h + i));
    }
#pragma unroll
    for (int i = 0; i < 17; ++i) put(17 * h + i, sum[i]);
  }
  return true;
}

// Wavefront W's whole K loop and epilogue (a template, so that the fifth
// tile's operand choice is static and every accumulator stays in place).
template <int W, bool G>
__device__ __forceinline__ void pd_body(const PdArgs& p, const PdSrc& src, PdLds& L, int lane, int64_t m0,
                                        int64_t n0, int nsteps, int xtile, int sl, int cnt) {
  f32x16_t acc[4][2], acc5[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[rt][0][e] = acc[rt][1][e] = acc5[rt][e] = 0.0f;
  }

  pd_issue<0>(p, src, m0, n0, 0, nsteps, L, 0, W);
  pd_issue<1>(p, src, m0, n0, 1, nsteps, L, 1, W);
  pd_issue<2>(p, src, m0, n0, 2, nsteps, L, 2, W);
  pd_issue<3>(p, src, m0, n0, 3, nsteps, L, 3, W);
  pd_wait_vmcnt<3 * kPdLX>();  // step 0 (and group 0) landed; steps 1..3 may be in flight
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  PdFrag f0, f1;
  pd_load_w<0, W>(L, 0, lane, f0);
  pd_load_x<0>(L, 0, lane, f0);
  pd_load_x<1>(L, 0, lane, f0);
  pd_load_x<2>(L, 0, lane, f0);
  pd_load_x<3>(L, 0, lane, f0);
  PdB bdec;
  pd_decode0(f0, lane >> 5, bdec);
  int xld = 4, xrd = 1;  // X stages of the next step to load into LDS / to read from LDS

  // Step t: wait for this wavefront's loads of step t + 1 (steps t + 2 and t + 3
  // may stay in flight: 2 x 4, plus 10 when one of them starts a group), meet
  // the barrier (after it every wavefront has finished step t - 1, so X stage
  // (t - 1) % 5 and, at a group start, the weight buffer of group t / 4 - 1 are
  // free), start the loads of step t + 4, read step t + 1's operands, and run
  // step t's MFMAs on the operands read during the previous step.  The raw
  // barrier has no fence, so the compiler adds no wait of its own.
#define PD_STEP(P, CUR, NXT)                                                          \
  {                                                                                  \
    const int t = tb + (P);                                                          \
    __builtin_amdgcn_sched_barrier(0);                                               \
    pd_wait_vmcnt_lds0<((P) == 0 || (P) == 3) ? 2 * kPdLX : 2 * kPdLX + kPdLW>();      \
    asm volatile("" ::: "memory");                                                   \
    __builtin_amdgcn_s_barrier();                                                    \
    asm volatile("" ::: "memory");                                                   \
    const PdDma dma = pd_dma_begin(p, m0, n0, t + 4, nsteps, L, xld);                \
    xld = pd_next_stage(xld);                                                        \
    pd_step<((P) + 1) & 3, W>(L, xrd, ((t + 1) >> 2) & 1, lane, CUR, NXT, bdec, acc, acc5, src, dma); \
    xrd = pd_next_stage(xrd);                                                        \
  }
  for (int tb = 0; tb < nsteps; tb += 4) {
    PD_STEP(0, f0, f1)
    PD_STEP(1, f1, f0)
    PD_STEP(2, f0, f1)
    PD_STEP(3, f1, f0)
  }
#undef PD_STEP
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the repeat loads past the end have landed

  // Fifth tile: add the wavefronts' partial sums in wavefront order; wavefront
  // W finishes row tile W.
  __syncthreads();
  // Only items 0..7 hold real columns (256 + 8 (v / 4) + 4h + v % 4 < 272).
  float4* red = reinterpret_cast<float4*>(&L.wg[0]);  // 4 x 4 x 2 x 64 lanes x 16 B = 32 KB of the weight groups
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    red[((W * 4 + rt) * 2 + 0) * 64 + lane] = make_float4(acc5[rt][0], acc5[rt][1], acc5[rt][2], acc5[rt][3]);
    red[((W * 4 + rt) * 2 + 1) * 64 + lane] = make_float4(acc5[rt][4], acc5[rt][5], acc5[rt][6], acc5[rt][7]);
  }
  __syncthreads();
  float4 t5a = red[((0 * 4 + W) * 2 + 0) * 64 + lane], t5b = red[((0 * 4 + W) * 2 + 1) * 64 + lane];
#pragma unroll
  for (int ww = 1; ww < 4; ++ww) {
    const float4 a = red[((ww * 4 + W) * 2 + 0) * 64 + lane], b = red[((ww * 4 + W) * 2 + 1) * 64 + lane];
    t5a.x += a.x; t5a.y += a.y; t5a.z += a.z; t5a.w += a.w;
    t5b.x += b.x; t5b.y += b.y; t5b.z += b.z; t5b.w += b.w;
  }

  if constexpr (!G) {
    if (cnt > 1 && !pd_exchange<W>(p, acc, t5a, t5b, xtile, sl, cnt, lane)) return;
  }

  // Epilogue: the BF16 tile goes through LDS (the X stages, free now) so that
  // the stores to Y are whole 16-byte pieces of rows.  Transposed 32x32 D
  // layout: item v of lane l is row l % 32 of Y's row tile and column
  // 8 (v / 4) + 4 (l / 32) + v % 4 of the column tile, so items 4q .. 4q + 3
  // are 4 consecutive columns (one 8-byte LDS write).
  const float ts = *p.tscale;
  const int l32 = lane & 31, h = lane >> 5;
  uint16_t* yt = reinterpret_cast<uint16_t*>(&L.xs[0]);  // [128][272] BF16, 69,632 bytes
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint2*>(yt + (32 * rt + l32) * kPdBN + 64 * W + 32 * c + 8 * q + 4 * h) =
            pd_pack4(acc[rt][c], 4 * q, ts);
  // Fifth tile: columns 256 + 8 (v / 4) + 4h + v % 4 exist for v < 8.
  *reinterpret_cast<uint2*>(yt + (32 * W + l32) * kPdBN + 256 + 4 * h) =
      make_uint2(pd_bf16x2(t5a.x * ts, t5a.y * ts), pd_bf16x2(t5a.z * ts, t5a.w * ts));
  *reinterpret_cast<uint2*>(yt + (32 * W + l32) * kPdBN + 264 + 4 * h) =
      make_uint2(pd_bf16x2(t5b.x * ts, t5b.y * ts), pd_bf16x2(t5b.z * ts, t5b.w * ts));
  __syncthreads();
  pd_store_tile<G>(p, yt, m0, n0, W * 64 + lane, L.rowmap);
}

// G: the grouped form over an expert stack.  Workgroup tile mt of the launch
// is tile mt of the sorted pair list: expert e with tile_off[e] <= mt <
// tile_off[e + 1], its rows 128 (mt - tile_off[e]) .. of that expert's pairs.
// Activation row of a pair = pair / topk, output row = pair; weights = matrix
// e.  Workgroups past the list's end zero the output rows of the pairs whose
// expert id is out of range (at least one m tile of them exists whenever such
// pairs do: the launch has ceil(pairs / 128) + E m tiles and the valid pairs
// use at most (V - nonempty experts) / 128 + nonempty experts of them), then
// exit.  In the grouped form p.m holds the number of pairs until the tile's
// row count replaces it.
// One tile over its K groups [g0, g1) (the whole K: 0, groups): sources from
// the tile's rows and columns, then the pipeline.  xtile / sl / cnt: the
// stream-K exchange (cnt = 1: none).  In the grouped form `tile` is the
// launch's tile id.
template <bool G>
__device__ __forceinline__ void pd_tile(PdArgs p, PdLds& L, int tid, int lane, int w, int tile, int g0, int g1,
                                        int xtile, int sl, int cnt) {
  const int nt = tile / p.m_tiles, mt = tile % p.m_tiles;
  int64_t m0 = (int64_t)mt * kPdBM;
  const int64_t n0 = (int64_t)nt * kPdBN;
  const int64_t kh = p.k >> 1, ks = p.k >> 4;  // row strides (the whole K)
  const int nsteps = 4 * (g1 - g0);
  // The sources start at group g0.
  p.x += (int64_t)g0 * kPdGroupK;
  p.packed += (int64_t)g0 * (kPdGroupK / 2);
  p.scales += (int64_t)g0 * (kPdGroupK / 16);

  PdSrc src;
  if constexpr (G) {
    const PdGroups gr = pd_groups(p);
    const int used = gr.tile_off[p.experts];
    if (mt >= used) {  // uniform per workgroup
      const int64_t cols = p.n - n0 < kPdBN ? p.n - n0 : kPdBN;
      for (int64_t i = gr.pair_off[p.experts] + (mt - used); i < p.m; i += p.m_tiles - used) {
        uint16_t* dst = p.y + (int64_t)gr.perm[i] * p.n + n0;
        for (int c = tid; c < cols; c += 256) dst[c] = 0;
      }
      return;
    }
    int lo = 0, hi = (int)p.experts;            // tile_off[lo] <= mt < tile_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (gr.tile_off[mid] <= mt) lo = mid; else hi = mid;
    }
    const int64_t base = gr.pair_off[lo] + (int64_t)(mt - gr.tile_off[lo]) * kPdBM;
    const int64_t rows = (int64_t)gr.pair_off[lo + 1] - base < kPdBM ? (int64_t)gr.pair_off[lo + 1] - base : kPdBM;
    if (tid < kPdBM) L.rowmap[tid] = gr.perm[base + (tid < rows ? tid : rows - 1)];  // read at the end
    // Per-lane offsets from x itself; rows past the tile's end repeat its last row.
#pragma unroll
    for (int i = 0; i < kPdLX; ++i) {
      const int q = w + 4 * i, r = 8 * q + (lane >> 3);
      const int64_t tok = gr.perm[base + (r < rows ? r : rows - 1)] / p.topk;
      src.x[i] = (uint32_t)(tok * p.k * 2 + 16 * ((lane & 7) ^ (r & 7)));
    }
    p.m = rows;
    p.packed += (int64_t)lo * p.w_stride;
    p.scales += (int64_t)lo * (p.w_stride >> 3);
    p.tscale += lo;
    m0 = 0;
  } else {
    // Per-lane offsets; rows past m or n repeat the last valid row (never stored).
#pragma unroll
    for (int i = 0; i < kPdLX; ++i) {
      const int q = w + 4 * i, r = 8 * q + (lane >> 3);
      const int64_t gm = m0 + r < p.m ? r : p.m - 1 - m0;
      src.x[i] = (uint32_t)(gm * p.k * 2 + 16 * ((lane & 7) ^ (r & 7)));
    }
  }
  src.wscale = 0;
#pragma unroll
  for (int i = 0; i < kPdLW; ++i) {
    const int q0 = 64 * (w + 4 * i), slot = (q0 < kPdWLast ? q0 : kPdWLast) + lane;
    const int r = slot / kPdWSlots, piece = slot - r * kPdWSlots;
    const int64_t gn = n0 + r < p.n ? n0 + r : p.n - 1;
    src.w[i] = piece < 8 ? p.packed + gn * kh + 16 * piece : p.scales + gn * ks;
    src.wscale |= (uint32_t)(piece == 8) << i;
  }

  switch (w) {
    case 0: pd_body<0, G>(p, src, L, lane, m0, n0, nsteps, xtile, sl, cnt); break;
    case 1: pd_body<1, G>(p, src, L, lane, m0, n0, nsteps, xtile, sl, cnt); break;
    case 2: pd_body<2, G>(p, src, L, lane, m0, n0, nsteps, xtile, sl, cnt); break;
    default: pd_body<3, G>(p, src, L, lane, m0, n0, nsteps, xtile, sl, cnt); break;
  }
}

template <bool G>
__global__ void __launch_bounds__(256) prefill_dma_kernel(PdArgs p) {
  __shared__ PdLds L;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  // Workgroups are dispatched to the 8 XCDs round-robin by id, so consecutive
  // logical ids of one XCD cover all m tiles of consecutive n tiles (the
  // weight tile is then fetched into that XCD's L2 once), and the slices of a
  // split tile sit on one XCD.  The whole tiles come first in the launch (the
  // split ones fill the round after them), each part remapped on its own.
  const int nwg = (int)gridDim.x, b = (int)blockIdx.x;
  const int groups = (int)(p.k / kPdGroupK);
  const int nwhole = (G || p.sk_tail == 0) ? nwg : p.sk_dp;
  if (b < nwhole) {
    int id = b;
    if ((nwhole & 7) == 0) id = (b & 7) * (nwhole >> 3) + (b >> 3);
    pd_tile<G>(p, L, tid, lane, w, id, 0, groups, 0, 0, 1);
    return;
  }
  if constexpr (!G) {
    // A slice of a split tile: split tile xt, slice sl of sk_c, groups [g0, g1).
    const int nb = nwg - nwhole;
    int j = b - nwhole;
    if ((nb & 7) == 0) j = (j & 7) * (nb >> 3) + (j >> 3);
    const int xt = j / p.sk_c, sl = j - xt * p.sk_c;
    const int g0 = (int)((int64_t)sl * groups / p.sk_c), g1 = (int)((int64_t)(sl + 1) * groups / p.sk_c);
    pd_tile<false>(p, L, tid, lane, w, p.sk_dp + xt, g0, g1, xt, sl, p.sk_c);
  }
}

}  // namespace

// The per-lane load offsets are 32-bit: a 128-row activation tile (256 k
// bytes) must stay below 4 GiB.
bool prefill_dma_supported(int64_t m, int64_t n, int64_t k) {
  return m > 0 && n > 0 && k > 0 && k % kPdGroupK == 0 && k < ((int64_t)1 << 24);
}

// Split plan for a tile count that leaves CUs idle:
//   * at most 128 tiles: every tile split into min(4, 256 / tiles) slices, so
//     that the workgroups stay within one round of 256;
//   * q whole rounds of 256 tiles and r <= 128 more (the down projection
//     5120 x 17408 at M = 2048 has 304 = 256 + 48): the 256 q tiles whole, then
//     each of the r others in min(8, 256 / r) slices, so that the last round
//     is full of workgroups with a fraction of a tile's work each;
//   * otherwise none.
// Each slice at least one 256-element group; no plan when no tile is split.
PdSplit prefill_split(int64_t m, int64_t n, int64_t k) {
  PdSplit sp;
  if (!prefill_dma_supported(m, n, k)) return sp;
  const int64_t tiles = ((n + kPdBN - 1) / kPdBN) * ((m + kPdBM - 1) / kPdBM), groups = k / kPdGroupK;
  const int64_t r = tiles % 256;
  int64_t dp, c;
  if (tiles <= 128) {
    dp = 0;
    c = 256 / tiles > 4 ? 4 : 256 / tiles;
  } else if (tiles > 256 && r > 0 && r <= 128) {
    dp = tiles - r;
    c = 256 / r > 8 ? 8 : 256 / r;
  } else {
    return sp;
  }
  c = c > groups ? groups : c;
  if (c < 2 || dp > ((int64_t)1 << 30)) return sp;
  sp.dp = (int)dp;
  sp.tail = (int)(tiles - dp);
  sp.c = (int)c;
  return sp;
}

int64_t prefill_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const PdSplit sp = prefill_split(m, n, k);
  if (sp.c < 2) return 0;
  return kSkinnyCounterBytes + (int64_t)sp.tail * sp.c * kPdPartBytes;
}

void launch_prefill_dma(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                        const uint8_t* scales, const float* tscale, uint16_t* y, void* workspace,
                        int64_t workspace_bytes, hipStream_t s) {
  const int64_t n_tiles = (n + kPdBN - 1) / kPdBN, m_tiles = (m + kPdBM - 1) / kPdBM;
  const int64_t need = prefill_workspace_bytes(m, n, k);
  if (need > 0 && workspace != nullptr && workspace_bytes >= need) {
    // Split tiles (at most 128, within the 4096 counters: one launch).  The
    // workspace starts with the arrival counters (zero, and left zero by every
    // launch), then the partial tiles.
    const PdSplit sp = prefill_split(m, n, k);
    const PdArgs a{x, m, n, k, packed, scales, tscale, y, (int)n_tiles, (int)m_tiles, nullptr, 0, 0, 0, sp.dp,
                   sp.tail, sp.c, reinterpret_cast<float*>(static_cast<char*>(workspace) + kSkinnyCounterBytes),
                   static_cast<uint32_t*>(workspace)};
    prefill_dma_kernel<false><<<dim3((unsigned)(sp.dp + sp.tail * sp.c)), 256, 0, s>>>(a);
    return;
  }
  // One launch covers up to 2^31 - 1 workgroups; larger m is split by row.
  const int64_t max_m_tiles = ((int64_t)1 << 30) / n_tiles;
  for (int64_t t0 = 0; t0 < m_tiles; t0 += max_m_tiles) {
    const int64_t mt = m_tiles - t0 < max_m_tiles ? m_tiles - t0 : max_m_tiles;
    const int64_t mm = (m - t0 * kPdBM) < mt * kPdBM ? (m - t0 * kPdBM) : mt * kPdBM;
    const PdArgs a{x + t0 * kPdBM * k, mm, n, k, packed, scales, tscale, y + t0 * kPdBM * n, (int)n_tiles, (int)mt,
                   nullptr, 0, 0, 0, 0, 0, 0, nullptr, nullptr};
    prefill_dma_kernel<false><<<dim3((unsigned)(n_tiles * mt)), 256, 0, s>>>(a);
  }
}

int64_t prefill_grouped_tile_bound(int64_t pairs, int64_t experts) { return (pairs + kPdBM - 1) / kPdBM + experts; }

// Activation offsets are 32-bit byte offsets from x; pair indices, tile
// counts and the workgroup id are int32.
bool prefill_grouped_supported(int64_t t_count, int64_t topk, int64_t experts, int64_t n, int64_t k) {
  if (t_count <= 0 || topk <= 0 || experts <= 0 || n <= 0 || k <= 0 || k % kPdGroupK != 0) return false;
  if (t_count > ((int64_t)1 << 31) / k || topk > ((int64_t)1 << 30) / t_count || experts > ((int64_t)1 << 28))
    return false;
  const int64_t n_tiles = (n + kPdBN - 1) / kPdBN;
  return n_tiles <= ((int64_t)1 << 31) / (prefill_grouped_tile_bound(t_count * topk, experts) + 1);
}

void launch_prefill_grouped(const uint16_t* x, int64_t topk, const int32_t* groups, int64_t pairs, int64_t experts,
                            int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales, const float* tscale,
                            uint16_t* y, hipStream_t s) {
  const int64_t n_tiles = (n + kPdBN - 1) / kPdBN, m_tiles = prefill_grouped_tile_bound(pairs, experts);
  const PdArgs a{x, pairs, n, k, packed, scales, tscale, y, (int)n_tiles, (int)m_tiles, groups, topk, experts,
                 n * (k >> 1), 0, 0, 0, nullptr, nullptr};
  prefill_dma_kernel<true><<<dim3((unsigned)(n_tiles * m_tiles)), 256, 0, s>>>(a);
}

}  // namespace nvfp4
