// MXFP4 tensors and the W4A4 (FP4 x FP4) GEMM on gfx950 (imp
// "docs/quantization.md", MXFP4 paragraph: the NVFP4 nibble layout with a
// UE8M0 micro-scale per 32 elements and no tensor scale, the format FP4
// matrix cores take natively, so an MXFP4 prefill runs at full FP4 rate).
//
// Format: packed [R, K/2] (element 2j in the low nibble of byte j), scales
// [R, K/32] UE8M0 (2^(e - 127)).  Quantizer (round to nearest, the OCP MX
// shared scale): per block of 32, E = clamp(floor(log2(amax)) - 2 + 127, 0,
// 254), code = sign | the E2M1 magnitude nearest to |v| / 2^(E - 127), ties to
// the even code, saturating at 6.
//
// GEMM: Y[M, N] (BF16) = Xq[M, K] . Wq[N, K]^T with
// v_mfma_scale_f32_32x32x64_f8f6f4 (both operands FP4 E2M1, UE8M0 scales per
// lane and 32-element block).  Lane l of an operand holds row l % 32 and 32
// consecutive K elements (16 bytes), with the scale byte of those 32 chosen by
// opsel from a 32-bit register; the output is the usual 32 x 32 FP32 tile.
// The weights are the A operand, so a lane ends up with 4 consecutive output
// columns of one row.  A workgroup (8 wavefronts, two per SIMD so that one
// issues MFMAs while the other waits) computes a 256 (n) x 256 (m) tile, each
// wavefront 128 (n) x 64 (m) (4 x 2 MFMA tiles, 128 accumulator registers).
// Per K chunk of 128 both operand tiles (256 rows x 64 bytes each) and their
// scale words (one 32-bit word per row: the chunk's four scale bytes) move from
// global memory to LDS with global_load_lds_dwordx4 / _dword, in a ring of four
// stages (three chunks in flight), in an XOR-swizzled layout that makes every
// fragment read conflict-free.
//
// K order inside a chunk: lane half h in MFMA K-step s (0, 1) takes the
// chunk's 32-element block 2s + h in both operands; its scale byte is byte
// 2s + h of the row's word, i.e. byte 2s (opsel) once the word is shifted
// right by 8h.
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {
namespace {

// ---------------------------------------------------------------------------
// Quantizer and dequantizer.
// ---------------------------------------------------------------------------

// E2M1 magnitude code of q >= 0 (exact): nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6;
// at a midpoint the even code wins (strict comparison against midpoints whose
// lower neighbour is even, >= for those whose upper neighbour is even);
// everything above 5 saturates at 6 (code 7).
__device__ __forceinline__ uint32_t mx_mag_code(float q) {
  return (uint32_t)(q > 0.25f) + (uint32_t)(q >= 0.75f) + (uint32_t)(q > 1.25f) + (uint32_t)(q >= 1.75f) +
         (uint32_t)(q > 2.5f) + (uint32_t)(q >= 3.5f) + (uint32_t)(q > 5.0f);
}

// Four lanes per 32-element block: lane q of the four loads elements
// [8q, 8q + 8) (16 bytes; a wavefront's load covers 1 KB of consecutive input),
// the block maximum comes from two lane exchanges, and lane q writes the code
// word of its 8 elements (a wavefront's store covers 256 consecutive bytes);
// lane 0 of the four writes the scale byte.
__global__ void __launch_bounds__(256) mx_quantize_kernel(const uint4* __restrict__ w, int64_t blocks,
                                                          uint32_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  // groups and the stride are multiples of 4 and the four lanes of a block are
  // consecutive, so they always take the same branches and the exchanges see
  // four live lanes.  Each thread loads four groups before it converts any.
  const int64_t groups = blocks * 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g0 < groups; g0 += 4 * stride) {
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t g = g0 + u * stride;
      q[u] = g < groups ? w[g] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t g = g0 + u * stride;
      if (g >= groups) continue;
      const uint32_t v[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = max(amax, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
      amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 64));
      amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2, 64));
      // floor(log2(amax)) = exponent field - 127 for a normal amax; E = that - 2 + 127.
      const int ef = (int)(amax >> 7);
      const int e = ef <= 2 ? 0 : (ef - 2 > 254 ? 254 : ef - 2);
      const float inv = __uint_as_float((uint32_t)(254 - e) << 23);  // 2^(127 - e), normal for e in [0, 252]
      uint32_t word = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t bits = (v[t / 2] >> (16 * (t & 1))) & 0xFFFFu;
        const float r = __uint_as_float((bits & 0x7FFFu) << 16) * inv;   // exact: a power-of-two scaling
        word |= (((bits >> 15) << 3) | mx_mag_code(r)) << (4 * t);
      }
      packed[g] = word;
      if ((g & 3) == 0) scales[g >> 2] = (uint8_t)e;
    }
  }
}

// Byte SEL of code word c (2 elements) times 2^(e - 127) as a BF16 pair.
template <int SEL>
__device__ __forceinline__ uint32_t mx_dq_pair(uint32_t c, int e) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, SEL);
  const float a = e == 255 ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(f[0], e - 127);
  const float b = e == 255 ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(f[1], e - 127);
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// One thread per 8 elements: a code word and its block's scale byte in, one
// 16-byte BF16 piece out (E2M1 * 2^(e - 127) is exact in FP32; one RNE to
// BF16; scale byte 0xFF gives NaN).
__global__ void __launch_bounds__(256) mx_dequant_kernel(const uint32_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ scales, int64_t pieces,
                                                         uint4* __restrict__ out) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < pieces; o += stride) {
    const uint32_t c = packed[o];
    const int e = scales[o >> 2];
    __builtin_nontemporal_store(u32x4_t{mx_dq_pair<0>(c, e), mx_dq_pair<1>(c, e), mx_dq_pair<2>(c, e),
                                        mx_dq_pair<3>(c, e)},
                                reinterpret_cast<u32x4_t*>(out) + o);
  }
}

// ---------------------------------------------------------------------------
// W4A4 GEMM.
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) const void mx_lds_t;

constexpr int kMxTile = 256;     // rows of W (n) and of X (m) per workgroup
constexpr int kMxKC = 128;       // K elements per chunk (64 bytes per row, 4 scale bytes per row)
constexpr int kMxRowPieces = 4;  // 16-byte pieces per row and chunk
constexpr int kMxStages = 4;     // the chunk in use and three in flight

// One chunk of both operands and their scale words.  Row r's logical piece p
// (elements [32 p, 32 p + 32) of the chunk) sits at physical piece
// p ^ ((r >> 1) & 3): a 128-bit read by 8 consecutive rows at one logical piece
// then covers all 32 banks.
struct MxStage {
  uint4 w[kMxTile * kMxRowPieces];  // 16 KB
  uint4 x[kMxTile * kMxRowPieces];  // 16 KB
  uint32_t sw[kMxTile];             // the chunk's 4 scale bytes of each weight row
  uint32_t sx[kMxTile];             // ... of each activation row
};

struct MxArgs {
  const uint8_t* xq;  // [M, K/2]
  const uint8_t* xs;  // [M, K/32]
  const uint8_t* wq;  // [N, K/2]
  const uint8_t* ws;  // [N, K/32]
  uint16_t* y;        // [M, N]
  int64_t m, n, k;
  int n_tiles, m_tiles;
};

template <typename U>
__device__ __forceinline__ uint32_t mx_lds_addr(const U* p) {
  return (uint32_t)(uintptr_t)(mx_lds_t*)p;
}

__device__ __forceinline__ uint64_t mx_uniform_ptr(const void* base) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
         (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
}

// One global_load_lds_dwordx4 (16 bytes per lane) / global_load_lds_dword (4
// bytes per lane) from base + off (uniform 64-bit base, per-lane 32-bit offset)
// to LDS lds + 16 * lane / lds + 4 * lane.  No register result; the kernel
// waits for them with explicit vmcnt waits (they are its only global loads in
// the K loop).
__device__ __forceinline__ void mx_lds_dma16(const void* base, uint32_t off, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(mx_uniform_ptr(base)), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void mx_lds_dma4(const void* base, uint32_t off, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("global_load_lds_dword %0, %1" ::"v"(off), "s"(mx_uniform_ptr(base)), "{m0}"(m0) : "memory");
}

template <int N>
__device__ __forceinline__ void mx_wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ i32x8_t mx_frag(uint4 v) { return i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0}; }

template <int OPSEL>
__device__ __forceinline__ void mx_mfma(f32x16_t& acc, const uint4& a, const uint4& b, uint32_t sa, uint32_t sb) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(mx_frag(a), mx_frag(b), acc, 4, 4, OPSEL, (int)sa, OPSEL,
                                                        (int)sb);
}

__device__ __forceinline__ uint32_t mx_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// MFMA K-step S (0, 1) of a chunk: lane half h takes the chunk's 32-element
// block 2S + h in both operands (logical piece 2S + h); its scale byte is
// byte 2S + h of the row's word, i.e. byte 2S once the word is shifted right
// by 8h.
template <int S, int NT>
__device__ __forceinline__ void mx_kstep(const MxStage& st, int wn, int wm, int lane, const uint32_t (&sw)[NT],
                                         const uint32_t (&sx)[2], f32x16_t (&acc)[NT][2]) {
  const int l32 = lane & 31, h = lane >> 5;
  uint4 a[NT], b[2];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int rw = 32 * NT * wn + 32 * t + l32;
    a[t] = st.w[rw * kMxRowPieces + ((2 * S + h) ^ ((rw >> 1) & 3))];
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int rx = 64 * wm + 32 * t + l32;
    b[t] = st.x[rx * kMxRowPieces + ((2 * S + h) ^ ((rx >> 1) & 3))];
  }
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) mx_mfma<2 * S>(acc[i][j], a[i], b[j], sw[i], sx[j]);
}

// Per wavefront and chunk: 2 + 2 operand DMA instructions (16 rows x 64 bytes
// each) and 1 scale-word instruction (64 rows x 4 bytes; wavefronts 0-3 the
// weights', 4-7 the activations'), 5 in all.  Chunks 0..2 are issued before the
// loop and chunk c + 3 at the top of chunk c (past the end: the last chunk
// again, into the stage chunk c - 1 used, which nothing reads any more), so at
// the top of chunk c exactly the newest 10 loads (chunks c + 1, c + 2) may
// still be in flight: vmcnt(10).
// TN: weight rows per workgroup tile, 256 or 192 (each wavefront TN / 2 of
// them: NT = TN / 64 MFMA tiles); the host picks the one whose grid fills the
// CUs best.  LDS stages always hold 256 weight rows; rows past TN repeat the
// tile's last row and are not used.
template <int TN>
__global__ void __launch_bounds__(512) mx_gemm_kernel(MxArgs p) {
  constexpr int NT = TN / 64;
  __shared__ MxStage stage[kMxStages];  // 4 x 34 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = w & 1, wm = w >> 1;  // wm 0..3: 64-row quarters of the m tile
  // Workgroups go to the 8 XCDs round-robin by id; when the count allows,
  // consecutive ids of one XCD take all m tiles of consecutive n tiles, so a
  // weight tile is fetched into that XCD's L2 once.
  const int nwg = p.n_tiles * p.m_tiles;
  int id = (int)blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int nt = id / p.m_tiles, mt = id % p.m_tiles;
  const int64_t n0 = (int64_t)nt * TN, m0 = (int64_t)mt * kMxTile;
  const int64_t kh = p.k >> 1, ks = p.k >> 5;
  const int nchunks = (int)(p.k / kMxKC), last = nchunks - 1;

  // Operand DMA: instruction i (of 16 per operand) fills LDS rows 16i .. 16i + 15;
  // this wavefront issues i = w + 8j.  Lane l: row 16i + l / 4, physical piece
  // l % 4, holding logical piece (l % 4) ^ ((row >> 1) & 3).  Rows past N or M
  // repeat the last row (their results are not stored).
  uint32_t offw[2], offx[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * (w + 8 * j) + (lane >> 2), pc = (lane & 3) ^ ((r >> 1) & 3);
    const int rn = r < TN ? r : TN - 1;
    const int64_t gn = n0 + rn < p.n ? n0 + rn : p.n - 1, gm = m0 + r < p.m ? m0 + r : p.m - 1;
    offw[j] = (uint32_t)(gn * kh + 16 * pc);
    offx[j] = (uint32_t)(gm * kh + 16 * pc);
  }
  // Scale words: wavefront w fills rows 64 (w % 4) .. + 63 of the weights (w < 4)
  // or of the activations (w >= 4).
  const int w4 = w & 3;
  const int srt = 64 * w4 + lane < TN ? 64 * w4 + lane : TN - 1;
  const int64_t srn = n0 + srt < p.n ? n0 + srt : p.n - 1;
  const int64_t srm = m0 + 64 * w4 + lane < p.m ? m0 + 64 * w4 + lane : p.m - 1;
  const uint32_t soff = (uint32_t)((w < 4 ? srn : srm) * ks);

  auto issue = [&](int c, int sidx) {
    const uint8_t* bw = p.wq + (int64_t)c * (kMxKC / 2);
    const uint8_t* bx = p.xq + (int64_t)c * (kMxKC / 2);
    MxStage& sg = stage[sidx];
    const uint32_t lw = mx_lds_addr(&sg.w[0]), lx = mx_lds_addr(&sg.x[0]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      mx_lds_dma16(bw, offw[j], lw + 1024 * (w + 8 * j));
      mx_lds_dma16(bx, offx[j], lx + 1024 * (w + 8 * j));
    }
    if (w < 4) mx_lds_dma4(p.ws + 4 * c, soff, mx_lds_addr(&sg.sw[64 * w4]));
    else mx_lds_dma4(p.xs + 4 * c, soff, mx_lds_addr(&sg.sx[64 * w4]));
  };

  f32x16_t acc[NT][2];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  issue(0, 0);
  issue(last < 1 ? last : 1, 1);
  issue(last < 2 ? last : 2, 2);
  const int l32 = lane & 31, h = lane >> 5;
  for (int c = 0; c < nchunks; ++c) {
    // This wavefront's share of chunk c has landed; after the barrier every
    // wavefront's has, and every wavefront is done with chunk c - 1's stage.
    mx_wait_vmcnt<10>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(c + 3 <= last ? c + 3 : last, (c + 3) % kMxStages);
    const MxStage& st = stage[c % kMxStages];
    uint32_t sw[NT], sx[2];
#pragma unroll
    for (int t = 0; t < NT; ++t) sw[t] = st.sw[32 * NT * wn + 32 * t + l32] >> (8 * h);
#pragma unroll
    for (int t = 0; t < 2; ++t) sx[t] = st.sx[64 * wm + 32 * t + l32] >> (8 * h);
    mx_kstep<0, NT>(st, wn, wm, lane, sw, sx, acc);
    mx_kstep<1, NT>(st, wn, wm, lane, sw, sx, acc);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): the repeat loads past the end have landed

  // Epilogue: the BF16 tile goes through LDS (the stages, free now) so that
  // the stores to Y are whole rows.  D of MFMA tile (i, j) is W-rows x X-rows:
  // lane l holds X row 32 j + l % 32 and W rows 8 q + 4 h + 0..3 (items
  // 4q .. 4q + 3), i.e. 4 consecutive output columns of one output row (one
  // 8-byte LDS write).  LDS tile: [256 rows (m)][TN columns (n)] BF16, 16-byte
  // pieces XOR-swizzled by the row's low 3 bits (within aligned groups of 8).
  __syncthreads();
  uint16_t* yt = reinterpret_cast<uint16_t*>(&stage[0]);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 64 * wm + 32 * j + l32;
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = 32 * NT * wn + 32 * i + 8 * q + 4 * h;         // multiple of 4
        const int piece = (col >> 3) ^ (r & 7), half = (col >> 2) & 1;  // 16-byte piece, 8-byte half
        const f32x16_t& a = acc[i][j];
        *reinterpret_cast<uint2*>(yt + r * TN + 8 * piece + 4 * half) =
            make_uint2(mx_bf16x2(a[4 * q], a[4 * q + 1]), mx_bf16x2(a[4 * q + 2], a[4 * q + 3]));
      }
  }
  __syncthreads();
  // 256 rows x TN / 8 pieces of 16 bytes; thread t takes pieces t, t + 512, ...:
  // consecutive threads write consecutive pieces of a row.  Nontemporal: Y is
  // not read again by this kernel.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int64_t rows = p.m - m0 < kMxTile ? p.m - m0 : kMxTile;
  const int64_t cols = p.n - n0 < TN ? p.n - n0 : TN;
  const bool vec = (p.n & 7) == 0 && ((uintptr_t)p.y & 15) == 0;
#pragma unroll 4
  for (int pi = tid; pi < kMxTile * (TN / 8); pi += 512) {
    const int r = pi / (TN / 8), c8 = 8 * (pi - r * (TN / 8));
    if (r >= rows || c8 >= cols) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(yt + r * TN + 8 * ((c8 >> 3) ^ (r & 7)));
    uint16_t* dst = p.y + (m0 + r) * p.n + n0 + c8;
    if (vec && c8 + 8 <= cols) {
      __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(dst));
    } else {
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
      for (int t = 0; t < 8 && c8 + t < cols; ++t) dst[t] = e[t];
    }
  }
}

unsigned mx_grid(int64_t items) {
  const int64_t b = (items + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

}  // namespace

void launch_mx_quantize(const uint16_t* w, int64_t rows, int64_t k, uint8_t* packed, uint8_t* scales, hipStream_t s) {
  const int64_t blocks = rows * (k / 32);
  mx_quantize_kernel<<<mx_grid(blocks), 256, 0, s>>>(reinterpret_cast<const uint4*>(w), blocks,
                                                         reinterpret_cast<uint32_t*>(packed), scales);
}

void launch_mx_dequant(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, uint16_t* out,
                       hipStream_t s) {
  const int64_t pieces = rows * (k / 8);
  mx_dequant_kernel<<<mx_grid(pieces), 256, 0, s>>>(reinterpret_cast<const uint32_t*>(packed), scales, pieces,
                                                    reinterpret_cast<uint4*>(out));
}

bool mx_gemm_supported(int64_t m, int64_t n, int64_t k) {
  return m > 0 && n > 0 && k > 0 && k % kMxKC == 0 && m * (k / 2) < ((int64_t)1 << 32) &&
         n * (k / 2) < ((int64_t)1 << 32) && ((n + 191) / 192) * ((m + kMxTile - 1) / kMxTile) < (1 << 30);
}

// The tile width whose grid fills the CUs best: time ~ rounds of the grid over
// the CUs x one tile's time (one workgroup per CU at a time).  Measured on the
// 17408 x 5120 weight, a 192-row tile takes 0.86 of a 256-row tile's time (not
// 0.75: the fixed costs per chunk stay), hence the weights 220 and 256.  The CU
// count is read once (the library runs on gfx950 devices, which all report the
// same).
static int mx_pick_tn(int64_t m, int64_t n) {
  static int cus = 0;
  if (cus == 0) {
    int d = 0, c = 0;
    cus = (hipGetDevice(&d) == hipSuccess &&
           hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, d) == hipSuccess && c > 0)
              ? c
              : 256;
  }
  const int64_t mt = (m + kMxTile - 1) / kMxTile;
  int best = 256;
  int64_t best_cost = INT64_MAX;
  for (int tn : {256, 192}) {
    const int64_t tiles = ((n + tn - 1) / tn) * mt, rounds = (tiles + cus - 1) / cus;
    const int64_t cost = rounds * (tn == 192 ? 220 : 256);
    if (cost < best_cost) {
      best_cost = cost;
      best = tn;
    }
  }
  return best;
}

void launch_mx_gemm(const uint8_t* xq, const uint8_t* xs, int64_t m, const uint8_t* wq, const uint8_t* ws, int64_t n,
                    int64_t k, uint16_t* y, hipStream_t s) {
  const int tn = mx_pick_tn(m, n);
  const int64_t n_tiles = (n + tn - 1) / tn, m_tiles = (m + kMxTile - 1) / kMxTile;
  const MxArgs a{xq, xs, wq, ws, y, m, n, k, (int)n_tiles, (int)m_tiles};
  if (tn == 192) mx_gemm_kernel<192><<<dim3((unsigned)(n_tiles * m_tiles)), 512, 0, s>>>(a);
  else mx_gemm_kernel<256><<<dim3((unsigned)(n_tiles * m_tiles)), 512, 0, s>>>(a);
}

}  // namespace nvfp4
