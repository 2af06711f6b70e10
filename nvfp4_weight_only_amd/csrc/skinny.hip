// Small-M (batched decode) W4A16 linear for gfx950.
//
// With a handful of activation rows (M <= 64) the linear is bound by the one
// pass over the packed weights (0.5625 B per weight element; model card
// "Qwen3.8-27B-NVFP4 (compressed-tensors)": weights NVFP4, activations BF16).
// This kernel streams every weight byte from HBM once, straight into
// registers, decodes it there into exact BF16 products E2M1 x E4M3, and feeds
// v_mfma_f32_16x16x32_bf16 with the weights as the A operand (16 weight rows)
// and the activations as the B operand (16 activation rows per MFMA tile).
// Every decoded weight fragment is used for all activation rows of the launch.
//
// Work split:
//   * a workgroup owns `rows` consecutive weight rows (T wavefronts of 16
//     rows) and one K slice made of whole 256-element chunks.  `rows` and the
//     number of slices are chosen on the host so that a launch is about one
//     workgroup per CU (68 rows x 1 slice for N = 17408; 80 rows x 4 slices
//     for N = 5120, K = 17408);
//   * the activation chunk (MT rows x 256 columns) is staged once per
//     workgroup in LDS, double-buffered, in MFMA fragment order;
//   * every wavefront keeps D chunks of its 16 weight rows in flight in
//     registers (D x 36 bytes per lane);
//   * with several K slices, every workgroup writes its FP32 partial sums to
//     the caller's workspace and bumps an arrival counter; the last
//     workgroup of a row block adds the slices in slice order (so the result
//     does not depend on arrival order), writes Y and resets the counter.
//
// K order inside a chunk: lane group g (lanes 16g .. 16g + 15) covers the
// chunk's columns [64g, 64g + 64); MFMA step j (0..7) takes its columns
// [64g + 8j, 64g + 8j + 8).  A lane thus reads 32 contiguous packed bytes and
// 4 contiguous scale bytes of its row per chunk, and the activation fragments
// follow the same order (a dot product does not depend on the order of its
// K terms; only the FP32 summation order changes).
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kSkChunk = 256;   // K elements per chunk
constexpr int kSkDepth = 6;     // weight chunks in flight per wavefront
// Ring stages of the streaming kernel by activation rows (D - 2 chunks in
// flight behind the one whose operands are being read).
constexpr int kSkRing8 = 5, kSkRing16 = 4, kSkRing32 = 4;

struct SkinnyArgs {
  const uint16_t* x;      // [m, k]
  int64_t m, n, k;
  const uint8_t* packed;  // [n, k/2]
  const uint8_t* scales;  // [n, k/16]
  const float* tscale;
  uint16_t* y;            // [m, n]
  float* part;            // [slices, m, npad] FP32 partial sums (slices > 1)
  uint32_t* count;        // [row_blocks, gridDim.y] arrival counters (slices > 1)
  int64_t npad;           // n rounded up to a multiple of 16
  int rows;               // weight rows per workgroup (a multiple of 4, <= 16 T)
  int slices;             // K slices (<= chunks)
  int chunks;             // ceil(k / 256)
};

// One chunk of one lane: 32 packed bytes (64 elements) and their 4 scales.
struct SkChunk {
  uint4 w0, w1;
  uint32_t s;
};

// LDS slot (16-byte units) of activation fragment (m-tile mt, MFMA step j,
// lane l).  The XOR keeps both the fragment reads (16 lanes of one l / 16 at a
// time) and the staging writes (16 consecutive K pieces of one row) free of
// bank conflicts.
__device__ __forceinline__ int sk_slot(int mt, int j, int l) { return ((mt * 8 + j) << 6) + (l ^ (j | ((l >> 1) & 8))); }

// Chunk c of a row whose K is a multiple of 256 (aligned 16-byte loads).
__device__ __forceinline__ void sk_load_w(const uint8_t* wrow, const uint8_t* srow, int c, int g, SkChunk& r) {
  const uint4* pw = reinterpret_cast<const uint4*>(wrow + (int64_t)c * 128 + 32 * g);
  r.w0 = pw[0];
  r.w1 = pw[1];
  r.s = *reinterpret_cast<const uint32_t*>(srow + (int64_t)c * 16 + 4 * g);
}

// Chunk c of a row for any K (a multiple of 16): one 16-element block at a
// time, blocks past the end of the row read as zero.
__device__ __forceinline__ void sk_load_w_any(const uint8_t* wrow, const uint8_t* srow, int c, int g, int kblocks,
                                              SkChunk& r) {
  uint32_t w[8], s = 0u;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int blk = c * 16 + 4 * g + b;
    const bool ok = blk < kblocks;
    const int cb = ok ? blk : 0;
    const uint2 v = *reinterpret_cast<const uint2*>(wrow + (int64_t)cb * 8);
    const uint32_t sv = srow[cb];
    w[2 * b] = ok ? v.x : 0u;
    w[2 * b + 1] = ok ? v.y : 0u;
    s |= (ok ? sv : 0u) << (8 * b);
  }
  r.w0 = make_uint4(w[0], w[1], w[2], w[3]);
  r.w1 = make_uint4(w[4], w[5], w[6], w[7]);
  r.s = s;
}

// 8 MFMA steps of one chunk: decode the lane's 8 packed words (scaled by their
// block's E4M3 scale) and multiply with every m-tile's activation fragment.
template <int NMT>
__device__ __forceinline__ void sk_compute(const SkChunk& r, const uint4* xb, int lane, f32x4_t* acc) {
  const float2 s01 = e4m3x2_to_f32<false>(r.s), s23 = e4m3x2_to_f32<true>(r.s);
  const uint32_t wd[8] = {r.w0.x, r.w0.y, r.w0.z, r.w0.w, r.w1.x, r.w1.y, r.w1.z, r.w1.w};
  const float sc[4] = {s01.x, s01.y, s23.x, s23.y};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, e2m1x8_scaled_to_bf16_hw(wd[j], sc[j >> 1]));
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xb[sk_slot(mt, j, lane)]);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mt], 0, 0, 0);
    }
  }
}

// Output of one 16-row tile (D layout of a 16x16 MFMA tile: acc[mt][r] is
// weight row tile_row + 4g + r, activation row m0 + 16 mt + lane % 16).
template <int NMT>
__device__ __forceinline__ void sk_store_y(const SkinnyArgs& p, const f32x4_t* acc, int64_t tile_row, int64_t row_end,
                                           int64_t m0, int lane) {
  const int64_t n0 = tile_row + 4 * (lane >> 4);
  const float t = *p.tscale;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int64_t gm = m0 + 16 * mt + (lane & 15);
    if (gm >= p.m || n0 >= row_end) continue;
    const f32x4_t v = acc[mt];
    uint16_t* yp = p.y + gm * p.n + n0;
    const uint32_t b0 = f32_to_bf16_rne(v[0] * t), b1 = f32_to_bf16_rne(v[1] * t);
    const uint32_t b2 = f32_to_bf16_rne(v[2] * t), b3 = f32_to_bf16_rne(v[3] * t);
    if ((p.n & 3) == 0 && n0 + 3 < row_end) {
      *reinterpret_cast<uint2*>(yp) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    } else {
      const uint32_t bb[4] = {b0, b1, b2, b3};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n0 + r < row_end) yp[r] = (uint16_t)bb[r];
    }
  }
}

// With several K slices: this slice's FP32 sums of one tile go to the
// workspace.  rows and row_start are multiples of 4, so a 4-row group is
// either wholly inside the block or starts past its end (the last block's
// padding columns n .. npad-1 may be written and are never read).  sk_arrive
// (splitk_arrive) orders these stores before the other slices' loads.
template <int NMT>
__device__ __forceinline__ void sk_publish(const SkinnyArgs& p, const f32x4_t* acc, int sl, int64_t tile_row,
                                           int64_t row_end, int64_t m0, int lane) {
  const int64_t n0 = tile_row + 4 * (lane >> 4);
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int64_t gm = m0 + 16 * mt + (lane & 15);
    if (gm < p.m && n0 < row_end) splitk_store_rows4(p.part + ((int64_t)sl * p.m + gm) * p.npad, n0, acc[mt]);
  }
}

// After every tile of the workgroup is published: true (in every thread) in the
// last workgroup of the row block to arrive, which then owns the reduction.
__device__ __forceinline__ bool sk_arrive(const SkinnyArgs& p, int rb, int tid) {
  (void)tid;
  return splitk_arrive(p.count + (int64_t)rb * gridDim.y + blockIdx.y, p.slices);
}

// In the last workgroup: one tile's slices added in slice order (this
// workgroup's own slice from registers), then written to y.
template <int NMT>
__device__ __forceinline__ void sk_reduce_tile(const SkinnyArgs& p, const f32x4_t* acc, int sl, int64_t tile_row,
                                               int64_t row_end, int64_t m0, int lane) {
  const int64_t n0 = tile_row + 4 * (lane >> 4);
  f32x4_t v[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    v[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t gm = m0 + 16 * mt + (lane & 15);
    if (gm >= p.m || n0 >= row_end) continue;
    for (int s = 0; s < p.slices; ++s) {
      v[mt] += s == sl ? acc[mt] : splitk_load_rows4(p.part + ((int64_t)s * p.m + gm) * p.npad, n0);
    }
  }
  sk_store_y<NMT>(p, v, tile_row, row_end, m0, lane);
}

// Epilogue of a kernel in which each wavefront owns one tile.
template <int NMT>
__device__ __forceinline__ void sk_epilogue(const SkinnyArgs& p, const f32x4_t* acc, int rb, int sl, int64_t tile_row,
                                            int64_t row_end, int64_t m0, int lane, int tid) {
  if (p.slices == 1) {
    sk_store_y<NMT>(p, acc, tile_row, row_end, m0, lane);
    return;
  }
  sk_publish<NMT>(p, acc, sl, tile_row, row_end, m0, lane);
  if (sk_arrive(p, rb, tid)) sk_reduce_tile<NMT>(p, acc, sl, tile_row, row_end, m0, lane);
}

template <int MT, int T, bool ALIGNED>
__global__ void __launch_bounds__(64 * T) skinny_kernel(SkinnyArgs p) {
  constexpr int NMT = MT / 16;
  constexpr int NT = 64 * T;
  constexpr int XPIECES = MT * (kSkChunk / 8);  // 16-byte activation pieces per chunk
  constexpr int XP = (XPIECES + NT - 1) / NT;
  constexpr int D = kSkDepth;
  __shared__ uint4 xs[2][NMT * 8 * 64];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
  const int rb = (int)(blockIdx.x / (unsigned)p.slices), sl = (int)(blockIdx.x % (unsigned)p.slices);
  const int64_t row_start = (int64_t)rb * p.rows;
  const int64_t row_end = row_start + p.rows < p.n ? row_start + p.rows : p.n;
  const int64_t m0 = (int64_t)blockIdx.y * MT;
  const int c0 = (int)((int64_t)sl * p.chunks / p.slices);
  const int nc = (int)((int64_t)(sl + 1) * p.chunks / p.slices) - c0;  // >= 1
  const int kblocks = (int)(p.k >> 4);

  // This lane's weight row (rows past the block's end repeat its last row; their
  // results are never stored).
  const int64_t tile_row = row_start + 16 * (tid >> 6);
  const int64_t wr = tile_row + (lane & 15) < row_end ? tile_row + (lane & 15) : row_end - 1;
  const uint8_t* wrow = p.packed + wr * (p.k >> 1);
  const uint8_t* srow = p.scales + wr * (p.k >> 4);
  auto w_load = [&](SkChunk& r, int ci) {
    if constexpr (ALIGNED)
      sk_load_w(wrow, srow, c0 + ci, g, r);
    else
      sk_load_w_any(wrow, srow, c0 + ci, g, kblocks, r);
  };

  // Activation staging: piece pc = (row pc / 32, 8 columns at 8 * (pc % 32)).
  uint4 xv[XP];
  auto x_load = [&](int ci) {
    const int64_t k0 = (int64_t)(c0 + ci) * kSkChunk;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int pc = tid + i * NT;
      const int64_t gm = m0 + (pc >> 5), gk = k0 + 8 * (pc & 31);
      const bool ok = pc < XPIECES && gm < p.m && gk < p.k;
      const uint4 v = *reinterpret_cast<const uint4*>(p.x + (ok ? gm * p.k + gk : 0));
      xv[i] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto x_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int pc = tid + i * NT;
      if (XPIECES % NT == 0 || pc < XPIECES) {
        const int ml = pc >> 5, q = pc & 31;
        xs[buf][sk_slot(ml >> 4, q & 7, (ml & 15) + 16 * (q >> 3))] = xv[i];
      }
    }
  };

  f32x4_t acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Prologue: weight chunks 0 .. D-1 (the last one repeated when the slice is
  // shorter), activation chunk 0 in LDS, activation chunk 1 in registers.
  SkChunk ring[D];
  x_load(0);
#pragma unroll
  for (int i = 0; i < D; ++i) w_load(ring[i], i < nc ? i : nc - 1);
  x_store(0);
  x_load(nc > 1 ? 1 : 0);
  __syncthreads();

  // One chunk: MFMAs on LDS buffer ci & 1, then the activations of chunk ci + 1
  // go to the other buffer, chunk ci + 2 is fetched, and (when `refill`) the
  // ring slot takes weight chunk ci + D.  The activation load is issued before
  // the weight refill so that waiting for it (one chunk later) does not wait
  // for the newest weight loads.
  auto step = [&](SkChunk& r, int ci, bool refill) {
    sk_compute<NMT>(r, xs[ci & 1], lane, acc);
    x_store((ci + 1) & 1);
    x_load(ci + 2 < nc ? ci + 2 : nc - 1);
    if (refill) w_load(r, ci + D);
    __syncthreads();
  };
  int cb = 0;
  for (; cb + 2 * D <= nc; cb += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) step(ring[i], cb + i, true);
  }
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (cb + i < nc) step(ring[i], cb + i, cb + i + D < nc);
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (cb + D + i < nc) step(ring[i], cb + D + i, false);

  sk_epilogue<NMT>(p, acc, rb, sl, tile_row, row_end, m0, lane, tid);
}

// ---------------------------------------------------------------------------
// Streaming kernel for K a multiple of 256 and up to 32 activation rows.
//
// Four wavefronts, one per SIMD.  Weights, scales and activations go from
// global memory straight into LDS with global_load_lds_dwordx4 (16 bytes per
// lane), through a ring of 4 chunk stages, so that every load instruction
// reads whole 128-byte lines and holds no registers:
//   * weights: 8 rows x 128 bytes (one chunk of 8 rows) per instruction;
//   * scales: 16 rows x 64 bytes (4 chunks) per instruction, once per 4 chunks,
//     into a double-buffered scale area;
//   * activations: 2 rows x 512 bytes per instruction, only the MX rows that
//     the launch can have (8, 16 or 32).
// The block has 4 row tiles of 16 (one per wavefront) or, for 68..80 rows, 5:
// the fifth tile's 8 MFMA steps per chunk are shared out 2 per wavefront and
// its partial sums are added in wavefront order at the end, so all four SIMDs
// do the same work.
//
// LDS layout (16-byte slots):
//   w: block row r, piece p (16 bytes = 32 elements) at slot 8 r + (p ^ ((r >> 1) & 7));
//   x: activation row m, piece q (8 elements) at slot 32 m + (q ^ (m & 15));
//   sg: row r's scales of chunk q of the group at slot 4 r + q.
// The XORs make the fragment reads conflict-free (16 lanes of one lane group
// read 16 rows at the same piece).
//
// Every wavefront issues the same number of load instructions for each chunk
// (spare slots repeat a real instruction and rewrite the same bytes), so the
// loads of a chunk are known to be complete at a fixed vmcnt.  The operand
// reads from LDS run one chunk ahead of the products: step c waits for chunk
// c + 1's loads, meets the barrier (after which every wavefront's share is in
// LDS), refills the stage of chunk c - 1 with chunk c + D - 1, issues the
// reads of chunk c + 1's operands and runs chunk c's MFMAs on the operands
// read in step c - 1, so the LDS reads overlap the decode.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) const void sk_lds_t;

// One global_load_lds_dwordx4: 16 bytes from each lane's `src` to LDS byte
// address lds + 16 * lane (lds wave-uniform, in M0).  Written out rather than
// through the compiler builtin: for the builtin, the compiler's wait insertion
// loses track of which stage a pending load writes at the loop head and waits
// for every load in flight (vmcnt(0)) once per ring turn, which drains the
// pipeline.  The instruction has no register result, so nothing the compiler
// allocates can be overwritten by the load in flight; the kernel's explicit
// vmcnt waits order the LDS reads after it.  M0 is declared clobbered, so the
// compiler keeps nothing of its own there across the statement.
__device__ __forceinline__ void sk_lds_dma16(const void* src, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);  // uniform per wavefront by construction
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(base) : "memory");
}

// The same with the nontemporal hint, for the weight rows: each instruction
// reads whole lines of data that no other workgroup reads.
__device__ __forceinline__ void sk_lds_dma16_nt(const void* src, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);  // uniform per wavefront by construction
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(base) : "memory");
}

template <typename U>
__device__ __forceinline__ uint32_t sk_lds_addr(const U* p) {
  return (uint32_t)(uintptr_t)(const sk_lds_t*)p;
}

template <int N>
__device__ __forceinline__ void sk_wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// vmcnt(N) and lgkmcnt(0): also this wavefront's LDS reads are done.
template <int N>
__device__ __forceinline__ void sk_wait_vmcnt_lds0() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// One ring stage: the block's weight rows and the MX activation rows of one
// chunk.
template <int MX, int TT>
struct SkStage {
  uint4 w[TT * 16 * 8];
  uint4 x[MX * 32];
};

// Scale groups (of 4 chunks) that start among chunks c + T0 .. c + D - 2,
// c % 4 == P.
constexpr int sk_groups_after(int P, int D, int T0 = 1) {
  int n = 0;
  for (int t = T0; t <= D - 2; ++t) n += ((P + t) % 4) == 0;
  return n;
}

// Per-lane global sources of one wavefront's loads, for chunk 0 (weights and
// activations) or scale group 0.
template <int LW, int LX, int LS>
struct SkDmaSrc {
  const uint8_t* w[LW];
  uint32_t wslot[LW];
  const uint16_t* x[LX];
  uint32_t xslot[LX];
  const uint8_t* s[LS];   // scales of chunk c0 + (lane % 4) of the group, clamped to the last chunk
  int64_t sclamp[LS];     // chunks past the end are read at this offset instead
  uint32_t sslot[LS];
};

// One chunk's MFMA operands as this wavefront reads them from LDS: its own
// tile (rows 16 w .. 16 w + 15 of the block) and, with FIVE, its two steps
// (2 w, 2 w + 1) of the fifth tile (block rows 64 .. 79; bytes [32 g + 8 w,
// + 8) of each row's chunk, i.e. half w % 2 of piece 2 g + w / 2, scale block
// 4 g + w).  Activation rows past MX (MX = 8 under a 16-wide tile) read row
// l15 % MX instead; they only feed output columns that are never stored.
template <int MT>
struct SkFrag {
  uint4 w0, w1;
  uint32_t sv;
  uint4 xb[8][MT / 16];
  uint2 wv5;
  uint32_t sv5;
  uint4 xb5[2][MT / 16];  // activation fragments of steps 2w and 2w + 1
};

template <int MT, int MX, int TT, bool FIVE>
__device__ __forceinline__ void sk_frag_read(SkFrag<MT>& F, const SkStage<MX, TT>& S, const uint4* sg, int q, int w,
                                             int r, int lane) {
  constexpr int NMT = MT / 16;
  const int g = lane >> 4, f = (r >> 1) & 7, l15 = lane & 15, xl = MX < 16 ? (l15 & (MX - 1)) : l15;
  F.w0 = S.w[r * 8 + ((2 * g) ^ f)];
  F.w1 = S.w[r * 8 + ((2 * g + 1) ^ f)];
  F.sv = reinterpret_cast<const uint32_t*>(&sg[4 * r + q])[g];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) F.xb[j][mt] = S.x[(16 * mt + xl) * 32 + ((8 * g + j) ^ xl)];
  if constexpr (FIVE) {
    const int r5 = 64 + l15, f5 = (r5 >> 1) & 7;
    F.wv5 = reinterpret_cast<const uint2*>(&S.w[r5 * 8 + ((2 * g + (w >> 1)) ^ f5)])[w & 1];
    F.sv5 = reinterpret_cast<const uint32_t*>(&sg[4 * r5 + q])[g];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) F.xb5[h][mt] = S.x[(16 * mt + xl) * 32 + ((8 * g + 2 * w + h) ^ xl)];
  }
}

// Decode and MFMAs of one chunk's operands; the MFMAs alternate between two
// accumulator chains (even and odd steps), summed once after the K loop.
template <int MT, bool FIVE>
__device__ __forceinline__ void sk_frag_compute(const SkFrag<MT>& F, int w, f32x4_t (*acc)[MT / 16], f32x4_t* acc5) {
  constexpr int NMT = MT / 16;
  const float2 s01 = e4m3x2_to_f32<false>(F.sv), s23 = e4m3x2_to_f32<true>(F.sv);
  const uint32_t wd[8] = {F.w0.x, F.w0.y, F.w0.z, F.w0.w, F.w1.x, F.w1.y, F.w1.z, F.w1.w};
  const float sc[4] = {s01.x, s01.y, s23.x, s23.y};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, e2m1x8_scaled_to_bf16_hw(wd[j], sc[j >> 1]));
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      acc[j & 1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, F.xb[j][mt]),
                                                               acc[j & 1][mt], 0, 0, 0);
  }
  if constexpr (FIVE) {
    const float sc5 = e4m3x2_to_f32<false>((F.sv5 >> (8 * w)) & 0xFFu).x;
    const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, e2m1x8_scaled_to_bf16_hw(F.wv5.x, sc5));
    const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, e2m1x8_scaled_to_bf16_hw(F.wv5.y, sc5));
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      acc5[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8_t, F.xb5[0][mt]), acc5[mt], 0, 0, 0);
      acc5[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8_t, F.xb5[1][mt]), acc5[mt], 0, 0, 0);
    }
  }
}

// Loads of chunk ci of the slice into stage S and, when ci % 4 == 0, of scale
// group ci / 4 into sg.  Past the slice, the slice's last chunk is loaded again
// (never read).
template <int MX, int TT, int LW, int LX, int LS>
__device__ __forceinline__ void sk_dma_issue(const SkinnyArgs& p, const SkDmaSrc<LW, LX, LS>& src, int ci, int nc,
                                             int c0, SkStage<MX, TT>& S, uint4* sg, int lane) {
  const int cc = ci < nc ? ci : nc - 1;
#pragma unroll
  for (int i = 0; i < LW; ++i) sk_lds_dma16_nt(src.w[i] + (int64_t)cc * 128, sk_lds_addr(&S.w[src.wslot[i]]));
#pragma unroll
  for (int i = 0; i < LX; ++i) sk_lds_dma16(src.x[i] + (int64_t)cc * kSkChunk, sk_lds_addr(&S.x[src.xslot[i]]));
  if ((ci & 3) == 0) {
#pragma unroll
    for (int i = 0; i < LS; ++i) {
      // this lane's chunk of the group; chunks past the weight's end read the last chunk's scales
      const bool in = (int64_t)(c0 + ci + (lane & 3)) < p.chunks;
      const uint8_t* a = in ? src.s[i] + (int64_t)ci * 16 : p.scales + src.sclamp[i];
      sk_lds_dma16(a, sk_lds_addr(&sg[src.sslot[i]]));
    }
  }
}

// MX: activation rows loaded per launch row (8, 16 or 32; the launch's m is at
// most MX, MFMA tiles cover MT >= MX rows and the rows past MX are never
// stored).  FIVE: the block has 5 row tiles (68..80 rows), else 4.  D: ring
// stages (D - 1 chunks in flight).
template <int MT, int MX, bool FIVE, int D>
__global__ void __launch_bounds__(256) skinny_dma_kernel(SkinnyArgs p) {
  constexpr int NMT = MT / 16;
  constexpr int TT = FIVE ? 5 : 4;
  constexpr int LW = FIVE ? 3 : 2;          // weight instructions per wavefront per chunk (2 per tile)
  constexpr int XI = MX / 2;                // activation instructions per chunk
  constexpr int LX = XI / 4;                // ... per wavefront (MX is a multiple of 8)
  constexpr int LS = FIVE ? 2 : 1;          // scale instructions per wavefront per group of 4 chunks
  constexpr int LB = LW + LX;               // loads per wavefront per chunk, scales aside
  // Scale buffers: group g + NB reuses g's buffer; it is issued with chunk
  // 4 (g + NB) at step 4 (g + NB) - (D - 1), after g's last read (issued at
  // step 4 g + 2, complete at step 4 g + 3's barrier).
  constexpr int NB = (D + 6) / 4;
  static_assert(4 * NB >= D + 2, "scale ring too short");
  static_assert(D >= 3, "one chunk in flight behind the one being read");
  static_assert(MX <= MT && (MX >= 16 || NMT == 1), "activation rows");
  typedef SkStage<MX, TT> Stage;
  __shared__ Stage st[D];
  __shared__ uint4 sgr[NB][TT * 16 * 4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rb = (int)(blockIdx.x / (unsigned)p.slices), sl = (int)(blockIdx.x % (unsigned)p.slices);
  const int64_t row_start = (int64_t)rb * p.rows;
  const int64_t row_end = row_start + p.rows < p.n ? row_start + p.rows : p.n;
  const int64_t m0 = (int64_t)blockIdx.y * MT;
  const int c0 = (int)((int64_t)sl * p.chunks / p.slices);
  const int nc = (int)((int64_t)(sl + 1) * p.chunks / p.slices) - c0;  // >= 1
  const int64_t kh = p.k >> 1, ks = p.k >> 4;

  // Per-lane sources.  Rows past the block's end, and activation rows past m,
  // repeat the last valid one (their results are never stored).
  SkDmaSrc<LW, LX, LS> src;
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int qi = (w + 4 * i) < 2 * TT ? (w + 4 * i) : 2 * TT - 1;  // 8-row instruction; spare slots repeat the last
    const int r = 8 * qi + (lane >> 3);
    const int64_t gr = row_start + r < row_end ? row_start + r : row_end - 1;
    src.w[i] = p.packed + gr * kh + (int64_t)c0 * 128 + 16 * ((lane & 7) ^ ((r >> 1) & 7));
    src.wslot[i] = 64 * qi;
  }
#pragma unroll
  for (int i = 0; i < LX; ++i) {
    const int J = w + 4 * i;
    const int ml = 2 * J + (lane >> 5);
    const int64_t gm = m0 + ml < p.m ? m0 + ml : p.m - 1;
    src.x[i] = p.x + gm * p.k + (int64_t)c0 * kSkChunk + 8 * ((lane & 31) ^ (ml & 15));
    src.xslot[i] = 64 * J;
  }
#pragma unroll
  for (int i = 0; i < LS; ++i) {
    const int ji = (w + 4 * i) < TT ? (w + 4 * i) : TT - 1;  // 16-row instruction; spare slots repeat the last
    const int r = 16 * ji + (lane >> 2);
    const int64_t gr = row_start + r < row_end ? row_start + r : row_end - 1;
    src.s[i] = p.scales + gr * ks + (int64_t)(c0 + (lane & 3)) * 16;
    src.sclamp[i] = gr * ks + (int64_t)(p.chunks - 1) * 16;
    src.sslot[i] = 64 * ji;
  }

  f32x4_t acc2[2][NMT], acc5[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) acc2[0][mt] = acc2[1][mt] = acc5[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int r = 16 * w + (lane & 15);

#pragma unroll
  for (int c = 0; c < D - 1; ++c)
    sk_dma_issue<MX, TT, LW, LX, LS>(p, src, c, nc, c0, st[c], sgr[(c >> 2) % NB], lane);
  // The operand reads run one chunk ahead of the products: step ci waits for
  // this wavefront's loads of chunk ci + 1 (chunks ci + 2 .. ci + D - 2 may
  // still be in flight: LB each, plus LS for each scale group that starts
  // among them) and for its own LDS reads of the previous step, meets the
  // barrier, refills the stage of chunk ci - 1 (read two steps ago) with chunk
  // ci + D - 1, reads chunk ci + 1's operands, and runs chunk ci's products on
  // the operands read in the previous step.  The raw barrier carries no
  // fence, so the compiler adds no wait of its own.
  SkFrag<MT> fa, fb;
  sk_wait_vmcnt_lds0<(D - 2) * LB + LS * sk_groups_after(0, D)>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  sk_frag_read<MT, MX, TT, FIVE>(fa, st[0], sgr[0], 0, w, r, lane);
  int si = 0;  // stage of chunk ci
#define SK_STEP(P, CUR, NXT)                                                                       \
  {                                                                                               \
    const int ci = cb + (P);                                                                      \
    if (ci < nc) {                                                                                \
      sk_wait_vmcnt_lds0<(D - 3) * LB + LS * sk_groups_after((P), D, 2)>();                       \
      asm volatile("" ::: "memory");                                                              \
      __builtin_amdgcn_s_barrier();                                                               \
      asm volatile("" ::: "memory");                                                              \
      /* with D == 4 the stage of chunk ci is P: constant offsets */                              \
      const int sc = D == 4 ? (P) : si;                                                           \
      const int cn = ci + D - 1, sn = sc == D - 1 ? 0 : sc + 1;                                   \
      sk_dma_issue<MX, TT, LW, LX, LS>(p, src, cn, nc, c0, st[sc == 0 ? D - 1 : sc - 1],          \
                                       sgr[(cn >> 2) % NB], lane);                                \
      sk_frag_read<MT, MX, TT, FIVE>(NXT, st[sn], sgr[((ci + 1) >> 2) % NB], ((P) + 1) & 3, w, r, lane); \
      sk_frag_compute<MT, FIVE>(CUR, w, acc2, acc5);                                              \
      si = sn;                                                                                    \
    }                                                                                             \
  }
  for (int cb = 0; cb < nc; cb += 4) {
    SK_STEP(0, fa, fb)
    SK_STEP(1, fb, fa)
    SK_STEP(2, fa, fb)
    SK_STEP(3, fb, fa)
  }
#undef SK_STEP
  // The refills past the slice are repeats that nothing reads; let them land
  // before the stages are reused below.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  f32x4_t acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) acc[mt] = acc2[0][mt] + acc2[1][mt];
  const int64_t tile_row = row_start + 16 * w;
  if constexpr (FIVE) {
    // Fifth tile: add the four wavefronts' partial sums in wavefront order.
    __syncthreads();  // every wavefront is past its last read of the stages
    f32x4_t* red = reinterpret_cast<f32x4_t*>(&st[0]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) red[(w * NMT + mt) * 64 + lane] = acc5[mt];
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        f32x4_t v = red[mt * 64 + lane];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) v += red[(ww * NMT + mt) * 64 + lane];
        acc5[mt] = v;
      }
    }
  }
  const int64_t row5 = row_start + 64;
  if (p.slices == 1) {
    sk_store_y<NMT>(p, acc, tile_row, row_end, m0, lane);
    if (FIVE && w == 0) sk_store_y<NMT>(p, acc5, row5, row_end, m0, lane);
    return;
  }
  sk_publish<NMT>(p, acc, sl, tile_row, row_end, m0, lane);
  if (FIVE && w == 0) sk_publish<NMT>(p, acc5, sl, row5, row_end, m0, lane);
  if (sk_arrive(p, rb, tid)) {
    sk_reduce_tile<NMT>(p, acc, sl, tile_row, row_end, m0, lane);
    if (FIVE && w == 0) sk_reduce_tile<NMT>(p, acc5, sl, row5, row_end, m0, lane);
  }
}

// ---------------------------------------------------------------------------
// Host side: launch shape.
// ---------------------------------------------------------------------------
struct SkinnyPlan {
  int mt = 16, t = 1, tiles = 1, rows = 16, slices = 1, chunks = 1;
  int64_t row_blocks = 1, gy = 1, npad = 0, count_bytes = 0, ws_bytes = 0;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

SkinnyPlan skinny_plan(int64_t m, int64_t n, int64_t k, bool split) {
  SkinnyPlan pl;
  pl.chunks = (int)ceil_div(k, kSkChunk);
  // K slices: aim at about 80 weight rows per workgroup and 256 workgroups.
  int64_t s = 1;
  if (split) {
    s = (80 * 256 + n / 2) / n;
    const int64_t cap = pl.chunks < 16 ? pl.chunks : 16;
    s = s < 1 ? 1 : (s > cap ? cap : s);
  }
  pl.slices = (int)s;
  // Rows per workgroup: one workgroup per CU (or per half CU, ... when that
  // needs more than 80 rows), a multiple of 4, at least one 16-row tile.
  int64_t per_cu = 1, rows = 0;
  for (;; ++per_cu) {
    rows = round_up(ceil_div(n * s, 256 * per_cu), 4);
    if (rows <= 80) break;
  }
  if (rows < 16) rows = 16;
  pl.rows = (int)rows;
  pl.tiles = (int)ceil_div(rows, 16);
  pl.t = pl.tiles <= 2 ? pl.tiles : (pl.tiles <= 4 ? 4 : 5);
  // Activation rows per launch row: up to 64, and at most 16 per wavefront
  // (keeps the register kernel's staging at <= 8 pieces per thread).
  pl.mt = m <= 16 ? 16 : (m <= 32 ? 32 : 64);
  while (pl.mt > 16 * pl.t) pl.mt /= 2;
  if (pl.mt == 64 && pl.t == 5) pl.t = 8;  // 64 activation rows on 5 wavefronts would spill registers
  pl.gy = ceil_div(m, pl.mt);
  pl.row_blocks = ceil_div(n, rows);
  pl.npad = round_up(n, 16);  // whole 16-row spans of partial sums (splitk_store_rows4)
  if (pl.slices > 1) {
    // The arrival counters sit in a region of fixed size at the start of the
    // workspace, the same for every shape, so that a workspace shared by
    // several shapes never finds one shape's partial sums where another keeps
    // its counters (every call leaves the counters it used at zero).
    if (pl.row_blocks * pl.gy * 4 > kSkinnyCounterBytes) return skinny_plan(m, n, k, false);
    pl.count_bytes = kSkinnyCounterBytes;
    pl.ws_bytes = pl.count_bytes + (int64_t)pl.slices * m * pl.npad * 4;
  }
  return pl;
}

// The streaming kernel takes K a multiple of 256 and m <= 32 (one launch row).
bool use_dma(const SkinnyPlan& pl, int64_t m, int64_t k) { return (k % kSkChunk) == 0 && m <= 32 && pl.gy == 1; }

template <int MT, int MX, int D>
void launch_dma(const SkinnyPlan& pl, const SkinnyArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(pl.row_blocks * pl.slices), 1u);
  if (pl.tiles == 5)
    skinny_dma_kernel<MT, MX, true, D><<<grid, 256, 0, s>>>(a);
  else
    skinny_dma_kernel<MT, MX, false, D><<<grid, 256, 0, s>>>(a);
}

template <int MT, int T>
void launch_reg_t(const SkinnyPlan& pl, const SkinnyArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(pl.row_blocks * pl.slices), (unsigned)pl.gy);
  if ((a.k & (kSkChunk - 1)) != 0)
    skinny_kernel<MT, T, false><<<grid, 64 * T, 0, s>>>(a);
  else
    skinny_kernel<MT, T, true><<<grid, 64 * T, 0, s>>>(a);
}

template <int MT>
void launch_reg(const SkinnyPlan& pl, const SkinnyArgs& a, hipStream_t s) {
  // The plan keeps MT <= 16 T; a wider workgroup than needed is also correct.
  switch (pl.t) {
    case 1:
      if constexpr (MT <= 16) return launch_reg_t<MT, 1>(pl, a, s);
      [[fallthrough]];
    case 2:
      if constexpr (MT <= 32) return launch_reg_t<MT, 2>(pl, a, s);
      [[fallthrough]];
    case 4: return launch_reg_t<MT, 4>(pl, a, s);
    case 5:
      if constexpr (MT <= 32) return launch_reg_t<MT, 5>(pl, a, s);
      [[fallthrough]];
    default: return launch_reg_t<MT, 8>(pl, a, s);
  }
}

}  // namespace

int64_t skinny_workspace_bytes(int64_t m, int64_t n, int64_t k) { return skinny_plan(m, n, k, true).ws_bytes; }

void launch_skinny(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                   const float* tscale, uint16_t* y, void* workspace, int64_t workspace_bytes, hipStream_t s) {
  SkinnyPlan pl = skinny_plan(m, n, k, true);
  if (pl.slices > 1 && (workspace == nullptr || workspace_bytes < pl.ws_bytes)) pl = skinny_plan(m, n, k, false);
  auto args = [&](int64_t mm0, int64_t mm) {
    SkinnyArgs a{x + mm0 * k, mm, n, k, packed, scales, tscale, y + mm0 * n, nullptr, nullptr, pl.npad,
                 pl.rows, pl.slices, pl.chunks};
    if (pl.slices > 1) {
      // Counters first, then the partial sums of this launch's rows.
      a.count = static_cast<uint32_t*>(workspace);
      a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.count_bytes) +
               (int64_t)pl.slices * mm0 * pl.npad;
    }
    return a;
  };
  if (use_dma(pl, m, k)) {
    const SkinnyArgs a = args(0, m);
    if (m <= 8)
      launch_dma<16, 8, kSkRing8>(pl, a, s);
    else if (m <= 16)
      launch_dma<16, 16, kSkRing16>(pl, a, s);
    else
      launch_dma<32, 32, kSkRing32>(pl, a, s);
    return;
  }
  // gridDim.y is limited to 65535 launch rows; larger m is split into launches.
  const int64_t max_gy = 65535;
  for (int64_t y0 = 0; y0 < pl.gy; y0 += max_gy) {
    const int64_t gy = pl.gy - y0 < max_gy ? pl.gy - y0 : max_gy;
    const int64_t mm0 = y0 * pl.mt, mm = (m - mm0) < gy * pl.mt ? (m - mm0) : gy * pl.mt;
    SkinnyPlan lp = pl;
    lp.gy = gy;
    const SkinnyArgs a = args(mm0, mm);
    switch (pl.mt) {
      case 16: launch_reg<16>(lp, a, s); break;
      case 32: launch_reg<32>(lp, a, s); break;
      default: launch_reg<64>(lp, a, s); break;
    }
  }
}

}  // namespace nvfp4
