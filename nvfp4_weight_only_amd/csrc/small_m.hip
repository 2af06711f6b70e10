// Small-M (batched decode, M <= 32) W4A16 linear on the kernel-native weight
// layout (nvfp4_prepare), gfx950.
//
// With a handful of activation rows the linear is bound by the one pass over
// the packed weights (0.5625 B per weight element; model card
// "Qwen3.8-27B-NVFP4 (compressed-tensors)": weights NVFP4, activations BF16;
// imp "docs/quantization.md", NVFP4 kernel pipeline: the decode path streams
// the packed weights once).  Every weight element is loaded from HBM once,
// straight into registers, decoded there to the exact BF16 value E2M1 x E4M3,
// and used as the A operand of v_mfma_f32_16x16x32_bf16 for all M activation
// rows at once (the activations are the B operand, 16 rows per MFMA tile).
//
// Kernel-native layout: 16-row tiles x 128-element quads, 1152 bytes per
// (tile, quad), quad-major (block (t, q) at (q * tiles + t) * 1152, so the
// tiles a workgroup reads for one quad are one contiguous run, and the eight
// wavefronts, on neighbouring quads, read neighbouring runs): 64 slots of 16
// bytes, slot 16 g + r holding the elements
// 32 i + 8 g .. + 8 (word i) of the quad in row r, then 32 scale words, word
// 16 h + r holding the scales of blocks 2 i + h (byte i) of row r.  A lane
// (r, g) of MFMA step 4 q + i takes word i of slot 16 g + r as its A operand
// (K order: step j covers [32 j, 32 j + 32), lane group g takes [32 j + 8 g,
// + 8) of both operands), and byte i of scale word 16 (g / 2) + r as its
// scale.  So a wavefront's weights of one (tile, quad) are one contiguous
// 1 KB load (whole cache lines) and its scales one 128-byte line; in the
// checkpoint layout the same data are 16 rows x 64 bytes and 16 rows x 8 bytes,
// twice and sixteen times the cache lines per byte.
//
// Work split.  A workgroup of eight wavefronts (two per SIMD) owns the output
// rows [row0, row0 + rows) (rows a multiple of 4) and one K slice of whole
// quads.  It reads the T tiles that cover its rows (a tile shared with the
// neighbouring block is read by both; their ids are consecutive on one XCD, so
// the second read is an L2 hit) and stores only its own rows.  The slice's
// quads are dealt out to the eight wavefronts in turn (wavefront w takes quads
// w, w + 8, ...), and every wavefront runs its quads for all T tiles, so the
// activation fragments of a quad are loaded once per wavefront and serve T
// tiles.  There is no barrier in the K loop: each
// wavefront double-buffers one quad of activation fragments and one quad of
// weights for all its tiles in registers, and issues the next quad's loads
// before the current quad's products.  At the end the eight wavefronts' FP32
// sums meet in LDS and are added in wavefront order.  With several K slices (a
// caller workspace), the workgroups of a row block exchange FP32 partial sums
// in the workspace and the last one to arrive adds them in slice order, so the
// result is the same bits on every run.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kSmWaves = 8;
constexpr int kSmQuadK = 128;
constexpr int kSmBlock = 1152;  // bytes per (tile, quad) of the kernel-native layout

struct SmArgs {
  const uint16_t* x;     // [m, k]
  int64_t m, n, k;
  const uint8_t* prep;   // kernel-native weight
  const float* tscale;
  uint16_t* y;           // [m, n]
  float* part;           // [slices, m, npad] FP32 partial sums (slices > 1), see splitk_store_rows4
  uint32_t* count;       // [row blocks] arrival counters (slices > 1)
  int64_t npad;          // n rounded up to a multiple of 16
  int rows;              // output rows per workgroup (a multiple of 4)
  int slices;            // K slices
  int quads;             // k / 128
  int xcd_order;         // 1: consecutive row blocks on one XCD (grid size a multiple of 8)
};

// One (tile, quad) as a lane holds it: its 16 packed bytes and its scale word.
struct SmW {
  uint4 w;
  uint32_t s;
};

// Activation fragments of one quad: step i, m tile mt.
template <int NMT>
struct SmX {
  uint4 v[4][NMT];
};

// tile: the tile's block of quad 0; qstride: bytes from one quad's blocks to
// the next (tiles * 1152, quad-major layout).
__device__ __forceinline__ void sm_load_w(SmW& r, const uint8_t* tile, int64_t qstride, int q, int lane) {
  const uint8_t* b = tile + (int64_t)q * qstride;
  r.w = ld_stream16(b + 16 * lane);
  r.s = ld_stream4(b + 1024 + 4 * (16 * ((lane >> 5) & 1) + (lane & 15)));
}

// Activation fragments of quad q: step i, m tile mt is row xr[mt] at elements
// [128 q + 32 i + 8 g, + 8).
template <int NMT>
__device__ __forceinline__ void sm_load_x(SmX<NMT>& r, const uint16_t* const* xr, int q, int g) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      r.v[i][mt] = *reinterpret_cast<const uint4*>(xr[mt] + (int64_t)q * kSmQuadK + 32 * i + 8 * g);
}

// Products of one quad of one row tile.
template <int NMT>
__device__ __forceinline__ void sm_quad(const SmW& r, const SmX<NMT>& xq, f32x4_t* acc) {
  const float2 s01 = e4m3x2_to_f32<false>(r.s), s23 = e4m3x2_to_f32<true>(r.s);
  const uint32_t wd[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
  const float sc[4] = {s01.x, s01.y, s23.x, s23.y};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, e2m1x8_scaled_to_bf16_hw(wd[i], sc[i]));
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, xq.v[i][mt]), acc[mt], 0, 0,
                                                        0);
  }
}

// Y of one (row tile, m tile) of the block: D layout of a 16x16 MFMA tile,
// item v of lane l is weight row tile_row + 4 (l / 16) + v and activation row
// gm = 16 mt + l % 16.  Only rows in [row0, row_end) belong to this block.
__device__ __forceinline__ void sm_store_y(const SmArgs& p, f32x4_t v, int64_t tile_row, int64_t row0,
                                           int64_t row_end, int64_t gm, int lane) {
  const int64_t n0 = tile_row + 4 * (lane >> 4);  // row0 and n0 are multiples of 4
  if (gm >= p.m || n0 < row0 || n0 >= row_end) return;
  const float t = *p.tscale;
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

// End of a small-M workgroup: the eight wavefronts' sums of each (row tile,
// m tile) pair meet in red (kSmWaves * T * NMT * 64 entries) and are added
// in wavefront order by wavefront pair % 8; then y, or with several K slices
// the workspace exchange.
template <int NMT, int T>
__device__ __forceinline__ void sm_finish(const SmArgs& p, f32x4_t (&acc)[T][NMT], f32x4_t* red, int w,
                                          int lane, int64_t tile0, int64_t row0, int64_t row_end, int rb,
                                          int sl) {
  constexpr int NP = T * NMT;  // (row tile, m tile) pairs
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) red[((w * T + t) * NMT + mt) * 64 + lane] = acc[t][mt];
  __syncthreads();
  constexpr int PPW = (NP + kSmWaves - 1) / kSmWaves;  // pairs per wavefront (1 or 2)
  f32x4_t sum[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int pi = w + kSmWaves * i;
    sum[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (pi < NP) {
#pragma unroll
      for (int ww = 0; ww < kSmWaves; ++ww) sum[i] += red[(ww * NP + pi) * 64 + lane];
    }
  }
  auto pair_rows = [&](int pi, int64_t& tile_row, int64_t& gm) {
    tile_row = (tile0 + pi / NMT) * 16;
    gm = 16 * (pi % NMT) + (lane & 15);
  };
  if (p.slices == 1) {
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int pi = w + kSmWaves * i;
      if (pi < NP) {
        int64_t tr, gm;
        pair_rows(pi, tr, gm);
        sm_store_y(p, sum[i], tr, row0, row_end, gm, lane);
      }
    }
    return;
  }

  // Several K slices: this slice's sums go to the workspace, then the
  // workgroups of the row block meet at the arrival counter (splitk_arrive);
  // the last one adds the slices in slice order and stores y.
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int pi = w + kSmWaves * i;
    if (pi < NP) {
      int64_t tr, gm;
      pair_rows(pi, tr, gm);
      const int64_t n0 = tr + 4 * (lane >> 4);
      if (gm < p.m && n0 >= row0 && n0 < row_end)
        splitk_store_rows4(p.part + ((int64_t)sl * p.m + gm) * p.npad, n0, sum[i]);
    }
  }
  if (!splitk_arrive(p.count + rb, p.slices)) return;
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int pi = w + kSmWaves * i;
    if (pi < NP) {
      int64_t tr, gm;
      pair_rows(pi, tr, gm);
      const int64_t n0 = tr + 4 * (lane >> 4);
      f32x4_t v = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if (gm < p.m && n0 >= row0 && n0 < row_end) {
        for (int s = 0; s < p.slices; ++s)
          v += s == sl ? sum[i] : splitk_load_rows4(p.part + ((int64_t)s * p.m + gm) * p.npad, n0);
      }
      sm_store_y(p, v, tr, row0, row_end, gm, lane);
    }
  }
}

// NMT: MFMA m tiles (16 activation rows each; rows past m repeat the last one
// and are never stored); T: tiles read per workgroup.
template <int NMT, int T>
__global__ void __launch_bounds__(64 * kSmWaves) small_m_kernel(SmArgs p) {
  constexpr int NP = T * NMT;  // (row tile, m tile) pairs
  __shared__ f32x4_t red[kSmWaves * NP * 64];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups are dispatched to the XCDs round-robin by id: with xcd_order,
  // logical block L of XCD x is x * (grid / 8) + id / 8, so consecutive row
  // blocks (which share a tile) run on one XCD.
  const unsigned id = blockIdx.x;
  const unsigned lid = p.xcd_order ? (id & 7u) * (gridDim.x >> 3) + (id >> 3) : id;
  const int rb = (int)(lid / (unsigned)p.slices), sl = (int)(lid % (unsigned)p.slices);
  const int64_t row0 = (int64_t)rb * p.rows;
  const int64_t row_end = row0 + p.rows < p.n ? row0 + p.rows : p.n;
  const int64_t tile0 = row0 >> 4;
  const int64_t tiles = (p.n + 15) >> 4;
  const int64_t qstride = tiles * kSmBlock;
  // This workgroup's quads [Q0, Q1); wavefront w takes every eighth of them,
  // Q0 + w, Q0 + w + 8, ..., so that the eight wavefronts read neighbouring
  // quads at any one time.
  const int Q0 = (int)((int64_t)sl * p.quads / p.slices), Q1 = (int)((int64_t)(sl + 1) * p.quads / p.slices);
  const int qw = Q0 + w;
  const int nq = Q1 > qw ? (Q1 - qw + kSmWaves - 1) / kSmWaves : 0;  // this wavefront's quads

  // Tiles past the weight's last tile repeat it (their rows are never stored).
  const uint8_t* tb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t ti = tile0 + t < tiles ? tile0 + t : tiles - 1;
    tb[t] = p.prep + ti * (int64_t)kSmBlock;
  }
  const uint16_t* xr[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int64_t mr = 16 * mt + (lane & 15);
    xr[mt] = p.x + (mr < p.m ? mr : p.m - 1) * p.k;
  }

  f32x4_t acc[T][NMT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  if (nq > 0) {
    // Double buffer: while quad j's products run, quad j + 1 is in flight.
    // Past the last quad the loads repeat it (in bounds; never used).  The
    // scheduling barrier keeps a quad's loads ahead of the previous quad's
    // products (the scheduler would otherwise sink them next to their uses to
    // save registers, and each quad would wait out a full load latency).
    SmX<NMT> xa, xb;
    SmW wa[T], wb[T];
    auto load = [&](SmX<NMT>& xq, SmW* wq, int j) {
      const int q = qw + kSmWaves * j;
      sm_load_x<NMT>(xq, xr, q, g);
#pragma unroll
      for (int t = 0; t < T; ++t) sm_load_w(wq[t], tb[t], qstride, q, lane);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto compute = [&](const SmX<NMT>& xq, const SmW* wq) {
#pragma unroll
      for (int t = 0; t < T; ++t) sm_quad<NMT>(wq[t], xq, acc[t]);
    };
    load(xa, wa, 0);
    int j = 0;
    for (; j + 1 < nq; j += 2) {
      load(xb, wb, j + 1);
      compute(xa, wa);
      load(xa, wa, j + 2 < nq ? j + 2 : nq - 1);
      compute(xb, wb);
    }
    if (j < nq) compute(xa, wa);
  }

  sm_finish<NMT, T>(p, acc, red, w, lane, tile0, row0, row_end, rb, sl);
}

// The same product with the activations staged through LDS.  Loaded straight
// into MFMA fragments, a quad's activations take 16 rows x 64 bytes (half
// cache lines) per instruction; here each wavefront copies its quad's MX rows
// x 256 bytes into its own LDS area with global_load_lds_dwordx4, four whole
// rows (eight cache lines) per instruction, and reads the fragments back with
// 16-byte LDS reads.  Slot s of row r holds the row's 16-byte piece s ^ (r %
// 16), so a fragment read (16 rows, one piece each) touches every 16-byte bank
// group once.  Two areas per wavefront: quad j + 1 is copied while quad j's
// products run.  Weights load into registers as above.  Only the wavefront
// reads its own area, so the K loop has no barrier; the wait for a quad's copy
// is a vmcnt that also covers its weight loads (loads complete in order).
typedef __attribute__((address_space(3))) const void sm_lds_t;

template <typename U>
__device__ __forceinline__ uint32_t sm_lds_addr(const U* ptr) {
  return (uint32_t)(uintptr_t)(const sm_lds_t*)ptr;
}

// 64 lanes x 16 bytes from per-lane global addresses to LDS bytes [lds, lds + 1024).
__device__ __forceinline__ void sm_lds_dma16(const void* src, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);  // uniform per wavefront by construction
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(base) : "memory");
}

template <int N>
__device__ __forceinline__ void sm_wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// MX: activation rows staged per quad (8, 16 or 32; m <= MX); T: tiles read
// per workgroup.
template <int MX, int T>
__global__ void __launch_bounds__(64 * kSmWaves) small_m_xl_kernel(SmArgs p) {
  constexpr int NMT = (MX + 15) / 16;
  constexpr int D = MX / 4;         // copy instructions per quad (four rows each)
  constexpr int XB = MX * 256;      // bytes of one quad's activations
  constexpr int RING = kSmWaves * 2 * XB;
  constexpr int RED = kSmWaves * T * NMT * 64 * 16;
  __shared__ uint4 lds[(RING > RED ? RING : RED) / 16];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const unsigned id = blockIdx.x;
  const unsigned lid = p.xcd_order ? (id & 7u) * (gridDim.x >> 3) + (id >> 3) : id;
  const int rb = (int)(lid / (unsigned)p.slices), sl = (int)(lid % (unsigned)p.slices);
  const int64_t row0 = (int64_t)rb * p.rows;
  const int64_t row_end = row0 + p.rows < p.n ? row0 + p.rows : p.n;
  const int64_t tile0 = row0 >> 4;
  const int64_t tiles = (p.n + 15) >> 4;
  const int64_t qstride = tiles * kSmBlock;
  const int Q0 = (int)((int64_t)sl * p.quads / p.slices), Q1 = (int)((int64_t)(sl + 1) * p.quads / p.slices);
  const int qw = Q0 + w;
  const int nq = Q1 > qw ? (Q1 - qw + kSmWaves - 1) / kSmWaves : 0;

  const uint8_t* tb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t ti = tile0 + t < tiles ? tile0 + t : tiles - 1;
    tb[t] = p.prep + ti * (int64_t)kSmBlock;
  }
  // Copy sources: instruction d, lane l covers row r = 4 d + l / 16 (rows past
  // m repeat row m - 1) and LDS slot l % 16, i.e. piece (l % 16) ^ (r % 16).
  const uint16_t* xsrc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int r = 4 * d + (lane >> 4);
    const int64_t gr = r < p.m ? r : p.m - 1;
    xsrc[d] = p.x + gr * p.k + 8 * ((lane & 15) ^ (r & 15));
  }
  // Fragment reads: step i, m tile mt is row rr = 16 mt + lane % 16 (rows past
  // m read row m - 1), piece 4 i + g, at slot (4 i + g) ^ (rr % 16).
  uint32_t xoff[4][NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    int rr = 16 * mt + (lane & 15);
    rr = rr < (int)p.m ? rr : (int)p.m - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) xoff[i][mt] = (uint32_t)(rr * 256 + (((4 * i + g) ^ (rr & 15)) * 16));
  }
  const uint32_t area = sm_lds_addr(&lds[0]) + (uint32_t)(w * 2 * XB);
  const char* lds_bytes = reinterpret_cast<const char*>(&lds[0]) + w * 2 * XB;

  f32x4_t acc[T][NMT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  if (nq > 0) {
    SmW wa[T], wb[T];
    auto load_w = [&](SmW* wq, int j) {
      const int q = qw + kSmWaves * j;
#pragma unroll
      for (int t = 0; t < T; ++t) sm_load_w(wq[t], tb[t], qstride, q, lane);
    };
    auto copy_x = [&](int j, int buf) {
      const int64_t q = qw + kSmWaves * j;
#pragma unroll
      for (int d = 0; d < D; ++d) sm_lds_dma16(xsrc[d] + q * kSmQuadK, area + (uint32_t)(buf * XB + d * 1024));
    };
    // Quad j: weights in wq, activations in area buf.  In issue order, quad
    // j's weight loads and copy precede quad j + 1's 2 T weight loads, so
    // vmcnt(2 T) after those means quad j has landed; quad j + 1's copy (into
    // the other area, whose reads finished in the previous step) follows.  The
    // empty asm statements with a memory clobber keep the loads above the
    // wait and the LDS reads below it.  Should the compiler split a weight load
    // into more instructions, the wait only gets stricter (loads complete in
    // order); it cannot issue fewer than one per load.
    auto step = [&](int j, const SmW* wq, SmW* wn, int buf) {
      if (j + 1 < nq) {
        load_w(wn, j + 1);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        sm_wait_vmcnt<2 * T>();
        __builtin_amdgcn_sched_barrier(0);
        copy_x(j + 1, buf ^ 1);
      } else {
        sm_wait_vmcnt<0>();
        asm volatile("" ::: "memory");
      }
      __builtin_amdgcn_sched_barrier(0);
      SmX<NMT> xq;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
          xq.v[i][mt] = *reinterpret_cast<const uint4*>(lds_bytes + buf * XB + xoff[i][mt]);
      __builtin_amdgcn_sched_barrier(0);  // all fragment reads in flight before the first product
#pragma unroll
      for (int t = 0; t < T; ++t) sm_quad<NMT>(wq[t], xq, acc[t]);
    };
    load_w(wa, 0);
    __builtin_amdgcn_sched_barrier(0);
    copy_x(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    int j = 0;
    for (; j + 1 < nq; j += 2) {
      step(j, wa, wb, 0);
      step(j + 1, wb, wa, 1);
    }
    if (j < nq) step(j, wa, wb, 0);
  }
  // Every copy has landed (the last step waited for all loads); the areas
  // become the reduction buffer once every wavefront is past its reads.
  __syncthreads();
  sm_finish<NMT, T>(p, acc, reinterpret_cast<f32x4_t*>(&lds[0]), w, lane, tile0, row0, row_end, rb, sl);
}

template <int MX>
void launch_xl(const SmallMPlan& pl, const SmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(pl.row_blocks * pl.slices));
  switch (pl.tiles) {
    case 1: small_m_xl_kernel<MX, 1><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
    case 2: small_m_xl_kernel<MX, 2><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
    case 3: small_m_xl_kernel<MX, 3><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
    case 4: small_m_xl_kernel<MX, 4><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
    default: small_m_xl_kernel<MX, 5><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
  }
}

// ---------------------------------------------------------------------------
// M = 1 on the kernel-native layout: a GEMV with the products on the vector
// ALU (the decode path of imp "docs/quantization.md", NVFP4 kernel pipeline:
// the packed weights streamed once, activations BF16).  A workgroup of W
// wavefronts owns T consecutive 16-row tiles; wavefront w takes the quads
// w, w + W, ... of all T tiles, in chunks of QW quads whose loads are all
// issued before the previous chunk's products (two chunks in registers).
//   * Weights: lane (r, g) = (lane % 16, lane / 16) loads slot lane of each
//     (tile, quad) block, i.e. word i = elements 32 i + 8 g .. + 8 of row r,
//     and the scale word 16 (g / 2) + r, whose byte i is the scale of the
//     block those elements lie in.  Each word is decoded to exact E2M1 values
//     (v_cvt_scalef32_pk_bf16_fp4 at scale 1), multiplied into the activations
//     by four v_dot2_f32_bf16, and the 8-element partial sum takes its E4M3
//     scale in one FMA: about 1.2 vector instructions per weight element.
//   * Activations: one 16-byte load per lane fetches the chunk's QW quads
//     (lane l: quad l / 16, piece l % 16) into the wavefront's own LDS area;
//     the products read them back as 16-byte broadcasts (16 lanes per
//     address), once per quad for all T tiles.  Only the wavefront itself
//     reads its area, so no barrier.
//   * The 64 lanes' sums meet over g by two shuffles, the W wavefronts' sums
//     in LDS in wavefront order, and y takes the tensor scale once.
// Rows past n are the layout's zero padding (tiles past the last repeat it)
// and are not stored.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float pg_dot8(uint32_t w, uint4 xv, float acc) {
  acc = dot2_bf16(e2m1x2_to_bf16<0>(w), xv.x, acc);
  acc = dot2_bf16(e2m1x2_to_bf16<1>(w), xv.y, acc);
  acc = dot2_bf16(e2m1x2_to_bf16<2>(w), xv.z, acc);
  return dot2_bf16(e2m1x2_to_bf16<3>(w), xv.w, acc);
}

template <int QW, int T>
struct PgChunk {
  uint4 x;         // activation piece: quad lane / 16 of the chunk, piece lane % 16
  SmW w[QW][T];    // weights and scales of the chunk's quads, per tile
};

template <int W, int T, int QW>
__global__ void __launch_bounds__(64 * W) gemv_prepared_kernel(const uint16_t* __restrict__ x, int64_t n, int quads,
                                                               const uint8_t* __restrict__ prep,
                                                               const float* __restrict__ tscale,
                                                               uint16_t* __restrict__ y) {
  static_assert(QW >= 1 && QW <= 4, "one activation load covers at most four quads");
  __shared__ uint4 xs[W][64];
  __shared__ float red[W][16 * T];
  const int lane = threadIdx.x & 63, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t tiles = (n + 15) >> 4, tile0 = (int64_t)blockIdx.x * T;
  const uint8_t* tb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) tb[t] = prep + (tile0 + t < tiles ? tile0 + t : tiles - 1) * (int64_t)kSmBlock;
  const int64_t qstride = tiles * kSmBlock;
  // This wavefront's quads w + W j, j < nq; chunk c holds j = QW c .. QW c + QW - 1.
  const int nq = quads > w ? (quads - w + W - 1) / W : 0;
  const int nc = (nq + QW - 1) / QW;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;
  if (nc > 0) {  // uniform per wavefront, taken before any load is in flight
    // Loads of chunk c; quads past the wavefront's last repeat it (never used).
    auto load = [&](PgChunk<QW, T>& ch, int c) {
      const int jx = QW * c + (lane >> 4);
      const int qx = w + W * ((lane >> 4) < QW && jx < nq ? jx : nq - 1);
      ch.x = *reinterpret_cast<const uint4*>(x + (int64_t)qx * kSmQuadK + 8 * (lane & 15));
#pragma unroll
      for (int j = 0; j < QW; ++j) {
        const int jj = QW * c + j, q = w + W * (jj < nq ? jj : nq - 1);
#pragma unroll
        for (int t = 0; t < T; ++t) sm_load_w(ch.w[j][t], tb[t], qstride, q, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto compute = [&](const PgChunk<QW, T>& ch, int c) {
      xs[w][lane] = ch.x;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < QW; ++j) {
        uint4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[i] = xs[w][16 * j + 4 * i + g];
        const bool valid = QW * c + j < nq;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const SmW& r = ch.w[j][t];
          const float2 s01 = e4m3x2_to_f32<false>(r.s), s23 = e4m3x2_to_f32<true>(r.s);
          float a = acc[t];
          a = fmaf(pg_dot8(r.w.x, xv[0], 0.0f), s01.x, a);
          a = fmaf(pg_dot8(r.w.y, xv[1], 0.0f), s01.y, a);
          a = fmaf(pg_dot8(r.w.z, xv[2], 0.0f), s23.x, a);
          a = fmaf(pg_dot8(r.w.w, xv[3], 0.0f), s23.y, a);
          acc[t] = valid ? a : acc[t];  // a select, not a branch: the next chunk's loads stay in flight
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();  // the area is rewritten by the next chunk
    };
    PgChunk<QW, T> ca, cb;
    load(ca, 0);
    int c = 0;
    for (; c + 1 < nc; c += 2) {
      load(cb, c + 1);
      compute(ca, c);
      load(ca, c + 2 < nc ? c + 2 : nc - 1);
      compute(cb, c + 1);
    }
    if (c < nc) compute(ca, c);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float v = acc[t];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (lane < 16) red[w][16 * t + lane] = v;
  }
  __syncthreads();
  const int tt = threadIdx.x;
  const int64_t row = tile0 * 16 + tt;
  if (tt < 16 * T && row < n) {
    float v = red[0][tt];
#pragma unroll
    for (int ww = 1; ww < W; ++ww) v += red[ww][tt];
    y[row] = (uint16_t)f32_to_bf16_rne(v * *tscale);
  }
}

// ---------------------------------------------------------------------------
// The kernel-native layout: conversion from the checkpoint layout and the
// dequantizer that reads it.
//
// Conversion: one wavefront per (tile, quad) block.  Lane (r, c) = (lane / 4,
// lane % 4) loads bytes 16 c .. 16 c + 16 of row 16 t + r's 64-byte quad
// segment: word g of those 16 bytes is word i = c of slot 16 g + r.  The words
// go through the wavefront's own LDS area to their slots, and lane u stores
// slot u: the block's first kilobyte in one 16-byte-per-lane instruction.
// Lanes 0..15 load row r's 8 scale bytes and store its two scale words
// (bytes 0, 2, 4, 6 and 1, 3, 5, 7).  A workgroup's four wavefronts take four
// consecutive quads of one tile, so the row segments they read complete each
// other's lines.  Rows past n are zero.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) prepare_kernel(const uint8_t* __restrict__ packed,
                                                      const uint8_t* __restrict__ scales, int64_t n, int64_t k,
                                                      uint8_t* __restrict__ out) {
  __shared__ uint32_t tr[4][256];  // per wavefront: word (row r, slot group g, word c) at (4 r + g) * 4 + c
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t tiles = (n + 15) >> 4, quads = k / kSmQuadK, kh = k >> 1, ks = k >> 4;
  const int64_t qgroups = (quads + 3) >> 2, jobs = tiles * qgroups;
  const int r = lane >> 2, c = lane & 3;
  for (int64_t job = blockIdx.x; job < jobs; job += gridDim.x) {
    const int64_t t = job / qgroups, q = 4 * (job - t * qgroups) + w;
    if (q >= quads) continue;  // uniform per wavefront; no workgroup barrier below
    const int64_t row = t * 16 + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < n) v = *reinterpret_cast<const uint4*>(packed + row * kh + q * 64 + 16 * c);
    tr[w][(4 * r + 0) * 4 + c] = v.x;
    tr[w][(4 * r + 1) * 4 + c] = v.y;
    tr[w][(4 * r + 2) * 4 + c] = v.z;
    tr[w][(4 * r + 3) * 4 + c] = v.w;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int g2 = lane >> 4, r2 = lane & 15;  // this lane's slot 16 g2 + r2
    const uint4 o = *reinterpret_cast<const uint4*>(&tr[w][(4 * r2 + g2) * 4]);
    uint8_t* blk = out + (q * tiles + t) * (int64_t)kSmBlock;
    *reinterpret_cast<uint4*>(blk + 16 * lane) = o;
    if (lane < 16) {
      const int64_t srow = t * 16 + lane;
      uint2 s8 = make_uint2(0u, 0u);
      if (srow < n) s8 = *reinterpret_cast<const uint2*>(scales + srow * ks + q * 8);
      uint32_t* sw = reinterpret_cast<uint32_t*>(blk + 1024);
      sw[lane] = __builtin_amdgcn_perm(s8.y, s8.x, 0x06040200u);
      sw[16 + lane] = __builtin_amdgcn_perm(s8.y, s8.x, 0x07050301u);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the area is rewritten by the next block
  }
}

// w = RNE_bf16(fl32(fl32(E2M1 * E4M3) * tscale)) for the 8 elements of one
// packed word and its E4M3 scale byte, as 8 BF16 in natural order.
__device__ __forceinline__ uint4 sm_dequant8(uint32_t p, uint32_t sbyte, float t) {
  return e2m1x8_dequant_bf16(p, e4m3x2_to_f32<false>(sbyte).x, t);
}

// One thread per packed slot: 32 elements of one row, four 16-byte stores.
__global__ void __launch_bounds__(256) dequant_prepared_kernel(const uint8_t* __restrict__ prep,
                                                               const float* __restrict__ tscale_p, int64_t n,
                                                               int64_t k, int64_t blocks, uint16_t* __restrict__ out) {
  const int64_t tiles = (n + 15) >> 4;
  const int64_t slots = blocks * 64;
  const float ts = *tscale_p;
  for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < slots;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = id >> 6, q = b / tiles, t = b - q * tiles;  // block b = q * tiles + t
    const int s = (int)(id & 63), g = s >> 4, r = s & 15;
    const int64_t row = t * 16 + r;
    if (row >= n) continue;
    const uint8_t* blk = prep + b * kSmBlock;
    const uint4 wv = *reinterpret_cast<const uint4*>(blk + 16 * s);
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(blk + 1024 + 4 * (16 * (g >> 1) + r));
    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
    uint16_t* dst = out + row * k + q * kSmQuadK + 8 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(dst + 32 * i) = sm_dequant8(wd[i], (sw >> (8 * i)) & 0xFFu, ts);
  }
}

template <int NMT>
void launch_nmt(const SmallMPlan& pl, const SmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(pl.row_blocks * pl.slices));
  switch (pl.tiles) {
    case 1: small_m_kernel<NMT, 1><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
    case 2: small_m_kernel<NMT, 2><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
    case 3: small_m_kernel<NMT, 3><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
    case 4: small_m_kernel<NMT, 4><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
    default: small_m_kernel<NMT, 5><<<grid, 64 * kSmWaves, 0, s>>>(a); break;
  }
}

int64_t sm_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t sm_round_up(int64_t a, int64_t b) { return sm_ceil_div(a, b) * b; }

unsigned sm_grid(int64_t items, int64_t max_blocks) {
  int64_t b = sm_ceil_div(items, 256);
  b = b > max_blocks ? max_blocks : b;
  return (unsigned)(b < 1 ? 1 : b);
}

// Most tiles any block of `rows` rows (a multiple of 4) covers: a block that
// starts r0 % 16 rows into a tile reaches ceil((r0 % 16 + rows) / 16) tiles, and
// r0 % 16 takes the values 0, 4, 8, 12 in a repeating pattern.
int64_t sm_max_tiles(int64_t n, int64_t rows) {
  int64_t worst = 0;
  for (int64_t b = 0; b < 4 && b * rows < n; ++b) {
    const int64_t r0 = b * rows, r1 = (r0 + rows < n ? r0 + rows : n) - 1;
    const int64_t t = r1 / 16 - r0 / 16 + 1;
    worst = t > worst ? t : worst;
  }
  return worst;
}

}  // namespace

int64_t prepared_bytes(int64_t n, int64_t k) { return sm_ceil_div(n, 16) * (k / kSmQuadK) * kSmBlock; }

void launch_prepare(const uint8_t* packed, const uint8_t* scales, int64_t n, int64_t k, uint8_t* out, hipStream_t s) {
  const int64_t jobs = sm_ceil_div(n, 16) * sm_ceil_div(k / kSmQuadK, 4);  // (tile, four quads) per workgroup
  prepare_kernel<<<(unsigned)(jobs < (1 << 20) ? jobs : (1 << 20)), 256, 0, s>>>(packed, scales, n, k, out);
}

void launch_dequant_prepared(const uint8_t* prep, const float* tscale, int64_t n, int64_t k, uint16_t* out,
                             hipStream_t s) {
  const int64_t blocks = sm_ceil_div(n, 16) * (k / kSmQuadK);
  dequant_prepared_kernel<<<sm_grid(blocks * 64, 1 << 20), 256, 0, s>>>(prep, tscale, n, k, blocks, out);
}

bool small_m_supported(int64_t m, int64_t n, int64_t k) {
  return m >= 1 && m <= 32 && n >= 1 && k >= kSmQuadK && k % kSmQuadK == 0 && k / kSmQuadK < (1 << 24);
}

SmallMPlan small_m_plan(int64_t m, int64_t n, int64_t k, bool split) {
  SmallMPlan pl;
  pl.quads = (int)(k / kSmQuadK);
  // K slices: about 80 weight rows per workgroup and 256 workgroups (one per
  // CU), each slice at least eight quads (one per wavefront), at most 16.
  // Each workgroup reads the activations of its K slice, so more slices mean
  // fewer activation bytes per CU, and more partial sums to exchange.  At the
  // down projection 5120 x 17408: M = 8, 80 rows x 4 slices 16.5 us against
  // 16.8 us for 40 x 2; M = 32, 26.9 us against 29.5 us.  With the exchange in
  // whole sectors (splitk_store_rows4): 15.6 / 21.1 us against 16.4 / 23.5 us
  // for 40 x 2, and 64 rows x 3 slices within 1 % (15.6 / 21.0 us).
  int64_t s = 1;
  if (split) {
    s = (80 * 256 + n / 2) / n;
    int64_t cap = pl.quads / kSmWaves;
    cap = cap < 16 ? cap : 16;
    s = s > cap ? cap : s;
    s = s < 1 ? 1 : s;
  }
  pl.slices = (int)s;
  // Rows per workgroup: at most 256 workgroups (one per CU; or per half CU,
  // ... when that needs more), a multiple of 4, covering at most five tiles.
  int64_t rows = 0;
  for (int64_t per_cu = 1;; ++per_cu) {
    const int64_t blocks = (256 * per_cu) / s;
    rows = sm_round_up(sm_ceil_div(n, blocks > 1 ? blocks : 1), 4);
    if (sm_max_tiles(n, rows) <= 5) break;
  }
  pl.rows = (int)rows;
  pl.tiles = (int)sm_max_tiles(n, rows);
  pl.row_blocks = sm_ceil_div(n, rows);
  pl.npad = sm_round_up(n, 16);  // whole 16-row spans of partial sums (splitk_store_rows4)
  if (pl.slices > 1) {
    if (pl.row_blocks * 4 > kSkinnyCounterBytes) return small_m_plan(m, n, k, false);
    pl.ws_bytes = kSkinnyCounterBytes + (int64_t)pl.slices * m * pl.npad * 4;
  }
  return pl;
}

template <int W, int T>
static void launch_pg(const uint16_t* x, int64_t n, int quads, const uint8_t* prep, const float* tscale, uint16_t* y,
                      hipStream_t s) {
  const int per_wave = (quads + W - 1) / W;  // quads of wavefront 0
  const dim3 grid((unsigned)sm_ceil_div(sm_ceil_div(n, 16), T));
  switch (per_wave < 4 ? per_wave : 4) {
    case 1: gemv_prepared_kernel<W, T, 1><<<grid, 64 * W, 0, s>>>(x, n, quads, prep, tscale, y); break;
    case 2: gemv_prepared_kernel<W, T, 2><<<grid, 64 * W, 0, s>>>(x, n, quads, prep, tscale, y); break;
    case 3: gemv_prepared_kernel<W, T, 3><<<grid, 64 * W, 0, s>>>(x, n, quads, prep, tscale, y); break;
    default: gemv_prepared_kernel<W, T, 4><<<grid, 64 * W, 0, s>>>(x, n, quads, prep, tscale, y); break;
  }
}

// Launch shape, from a sweep of wavefronts per workgroup (W = 1 .. 16) and
// tiles per workgroup (T = 1 .. 4), host-launched over rotated copies:
//   5120 x 5120: W 16, T 2 5.63 us (W 16, T 1 6.67; W 4, T 2 6.04);
//   34816 x 5120: W 4, T 1 19.46 us (W 16, T 1 25.8; W 10, T 1 21.5);
//   5120 x 17408: W 4, T 2 12.37 us (W 16, T 2 13.4; W 4, T 1 13.2).
// Many tiles: small workgroups, one tile each; few tiles and long K: small
// workgroups with two tiles; few tiles and short K: 16 wavefronts share K.
void launch_gemv_prepared(const uint16_t* x, int64_t n, int64_t k, const uint8_t* prep, const float* tscale,
                          uint16_t* y, hipStream_t s) {
  const int quads = (int)(k / kSmQuadK);
  const int64_t tiles = sm_ceil_div(n, 16);
  if (tiles >= 1024)
    launch_pg<4, 1>(x, n, quads, prep, tscale, y, s);
  else if (quads > 64)
    launch_pg<4, 2>(x, n, quads, prep, tscale, y, s);
  else
    launch_pg<16, 2>(x, n, quads, prep, tscale, y, s);
}

void launch_small_m(const SmallMPlan& pl, const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* prep,
                    const float* tscale, uint16_t* y, void* workspace, hipStream_t s) {
  const int64_t grid = pl.row_blocks * pl.slices;
  SmArgs a{x, m, n, k, prep, tscale, y, nullptr, nullptr, pl.npad, pl.rows, pl.slices, pl.quads, (grid & 7) == 0};
  if (pl.slices > 1) {
    a.count = static_cast<uint32_t*>(workspace);
    a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kSkinnyCounterBytes);
  }
  // m > 16: activations through LDS (128 KiB per workgroup, so only where the
  // plan has one workgroup per CU).  Measured against the register form on the
  // 17408 x 5120 and 5120 x 17408 weights: M = 32 17.8 / 24.1 us against 20.2 /
  // 27.7 us; at M = 8 the LDS form (8 rows) was slower, 13.7 / 16.4 against
  // 13.0 / 15.9 us.
  if (m > 16 && pl.row_blocks * pl.slices <= 256) {
    launch_xl<32>(pl, a, s);
  } else if (m <= 16) {
    launch_nmt<1>(pl, a, s);
  } else {
    launch_nmt<2>(pl, a, s);
  }
}

}  // namespace nvfp4
