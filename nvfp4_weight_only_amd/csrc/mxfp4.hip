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
// columns of one row.  A workgroup (4 wavefronts) computes a 256 (n) x 256 (m)
// tile, each wavefront 128 x 128 (4 x 4 MFMA tiles, all 256 AGPRs).  Per K
// chunk of 256 both operand tiles (256 rows x 128 bytes each) move from global
// memory to LDS with global_load_lds_dwordx4, double-buffered (128 KB), in an
// XOR-swizzled layout that makes every fragment read conflict-free.
//
// K order inside a chunk: lane half h in MFMA K-step s (0..3) takes elements
// [128 h + 32 s, 128 h + 32 s + 32) of the chunk, i.e. 32-element block 4h + s,
// for both operands (the dot product does not depend on the order of its
// terms).  A lane's four scale bytes of a chunk are then one aligned 32-bit
// word (blocks 4h .. 4h + 3), and K-step s selects byte s of it.
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

// One thread per 32-element block (64 input bytes in, 16 code bytes and one
// scale byte out).
__global__ void __launch_bounds__(256) mx_quantize_kernel(const uint4* __restrict__ w, int64_t blocks,
                                                          uint4* __restrict__ packed, uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < blocks; b += stride) {
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = w[4 * b + i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = max(amax, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
    // floor(log2(amax)) = exponent field - 127 for a normal amax; E = that - 2 + 127.
    const int ef = (int)(amax >> 7);
    const int e = ef <= 2 ? 0 : (ef - 2 > 254 ? 254 : ef - 2);
    const float inv = __uint_as_float((uint32_t)(254 - e) << 23);  // 2^(127 - e), a normal float for e in [0, 252]
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t bits = (v[4 * j + t / 2] >> (16 * (t & 1))) & 0xFFFFu;
        const float q = __uint_as_float((bits & 0x7FFFu) << 16) * inv;   // exact: a power-of-two scaling
        word |= (((bits >> 15) << 3) | mx_mag_code(q)) << (4 * t);
      }
      out[j] = word;
    }
    packed[b] = make_uint4(out[0], out[1], out[2], out[3]);
    scales[b] = (uint8_t)e;
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
constexpr int kMxKC = 256;       // K elements per chunk (128 bytes per row)
constexpr int kMxRowPieces = 8;  // 16-byte pieces per row and chunk

struct MxStage {
  uint4 w[kMxTile * kMxRowPieces];  // 32 KB
  uint4 x[kMxTile * kMxRowPieces];  // 32 KB
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

// One global_load_lds_dwordx4: 16 bytes per lane from base + off (uniform
// 64-bit base, per-lane 32-bit offset) to LDS lds + 16 * lane.  No register
// result; the kernel waits for it with an explicit vmcnt wait.
__device__ __forceinline__ void mx_lds_dma16(const void* base, uint32_t off, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t bs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(off), "s"(bs) : "memory");
}

__device__ __forceinline__ i32x8_t mx_frag(uint4 v) { return i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0}; }

template <int S>
__device__ __forceinline__ void mx_mfma(f32x16_t& acc, const uint4& a, const uint4& b, uint32_t sa, uint32_t sb) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(mx_frag(a), mx_frag(b), acc, 4, 4, S, (int)sa, S, (int)sb);
}

__device__ __forceinline__ uint32_t mx_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// The four K-steps of one chunk on stage `st`: fragments of row r, logical
// piece 4h + s at physical piece (4h + s) ^ (r & 7).
template <int S>
__device__ __forceinline__ void mx_kstep(const MxStage& st, int wn, int wm, int lane, const uint32_t (&sw)[4],
                                         const uint32_t (&sx)[4], f32x16_t (&acc)[4][4]) {
  const int l32 = lane & 31, h = lane >> 5;
  uint4 a[4], b[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int rw = 128 * wn + 32 * t + l32, rx = 128 * wm + 32 * t + l32;
    a[t] = st.w[rw * kMxRowPieces + ((4 * h + S) ^ (rw & 7))];
    b[t] = st.x[rx * kMxRowPieces + ((4 * h + S) ^ (rx & 7))];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) mx_mfma<S>(acc[i][j], a[i], b[j], sw[i], sx[j]);
}

__global__ void __launch_bounds__(256) mx_gemm_kernel(MxArgs p) {
  __shared__ MxStage stage[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = w & 1, wm = w >> 1;
  // Workgroups go to the 8 XCDs round-robin by id; when the count allows,
  // consecutive ids of one XCD take all m tiles of consecutive n tiles, so a
  // weight tile is fetched into that XCD's L2 once.
  const int nwg = p.n_tiles * p.m_tiles;
  int id = (int)blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int nt = id / p.m_tiles, mt = id % p.m_tiles;
  const int64_t n0 = (int64_t)nt * kMxTile, m0 = (int64_t)mt * kMxTile;
  const int64_t kh = p.k >> 1, ks = p.k >> 5;
  const int nchunks = (int)(p.k / kMxKC);

  // DMA sources: instruction i (of 32 per operand) fills LDS rows 8i .. 8i + 7;
  // this wavefront issues i = w + 4j.  Lane l: row 8i + l / 8, physical piece
  // l % 8, which holds logical piece (l % 8) ^ (row & 7).  Rows past M or N
  // repeat the last valid row (their results are not stored).
  uint32_t offw[8], offx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * (w + 4 * j) + (lane >> 3), q = lane & 7, pc = q ^ (r & 7);
    const int64_t gn = n0 + r < p.n ? n0 + r : p.n - 1, gm = m0 + r < p.m ? m0 + r : p.m - 1;
    offw[j] = (uint32_t)(gn * kh + 16 * pc);
    offx[j] = (uint32_t)(gm * kh + 16 * pc);
  }
  // Scale words: tile t of this wavefront, row 32 t + lane % 32, blocks 4h .. 4h + 3 of the chunk, as
  // 32-bit word offsets from the scale arrays (a scale array is below 2^28 words when its packed array
  // is below 2^32 bytes).
  const uint32_t* ws32 = reinterpret_cast<const uint32_t*>(p.ws);
  const uint32_t* xs32 = reinterpret_cast<const uint32_t*>(p.xs);
  uint32_t swo[4], sxo[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t rn = n0 + 128 * wn + 32 * t + (lane & 31), rm = m0 + 128 * wm + 32 * t + (lane & 31);
    swo[t] = (uint32_t)((rn < p.n ? rn : p.n - 1) * (ks >> 2) + (lane >> 5));
    sxo[t] = (uint32_t)((rm < p.m ? rm : p.m - 1) * (ks >> 2) + (lane >> 5));
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto issue = [&](int c, int sidx) {
    const uint8_t* bw = p.wq + (int64_t)c * (kMxKC / 2);
    const uint8_t* bx = p.xq + (int64_t)c * (kMxKC / 2);
    const uint32_t lw = mx_lds_addr(&stage[sidx].w[0]), lx = mx_lds_addr(&stage[sidx].x[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mx_lds_dma16(bw, offw[j], lw + 1024 * (w + 4 * j));
      mx_lds_dma16(bx, offx[j], lx + 1024 * (w + 4 * j));
    }
  };

  uint32_t sw[4], sx[4];
  issue(0, 0);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    sw[t] = ws32[swo[t]];
    sx[t] = xs32[sxo[t]];
  }
  for (int c = 0; c < nchunks; ++c) {
    // Chunk c's operands (and scale words) have landed in every wavefront;
    // after the barrier every wavefront is done with chunk c - 1's stage.
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Always issued (past the end: the last chunk again, into the stage nothing
    // reads any more): loads under a branch would end in a full drain at the join.
    const int cn = c + 1 < nchunks ? c + 1 : c;
    issue(cn, (c + 1) & 1);
    uint32_t nsw[4], nsx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      nsw[t] = ws32[swo[t] + 2 * cn];
      nsx[t] = xs32[sxo[t] + 2 * cn];
    }
    const MxStage& st = stage[c & 1];
    mx_kstep<0>(st, wn, wm, lane, sw, sx, acc);
    mx_kstep<1>(st, wn, wm, lane, sw, sx, acc);
    mx_kstep<2>(st, wn, wm, lane, sw, sx, acc);
    mx_kstep<3>(st, wn, wm, lane, sw, sx, acc);
    // The copy below uses the next chunk's scale loads: kept behind the MFMAs
    // (hoisted above them, its wait would stall the chunk for a load latency).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sw[t] = nsw[t];
      sx[t] = nsx[t];
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): the repeat loads past the end have landed

  // Epilogue: the BF16 tile goes through LDS (the stages, free now) so that
  // the stores to Y are whole rows.  D of MFMA tile (i, j) is W-rows x X-rows:
  // lane l holds X row 32 j + l % 32 and W rows 8 q + 4 h + 0..3 (items
  // 4q .. 4q + 3), i.e. 4 consecutive output columns of one output row (one
  // 8-byte LDS write).  LDS tile: [256 rows (m)][256 columns (n)] BF16, row
  // stride 512 bytes, 16-byte pieces XOR-swizzled by the row's low 3 bits.
  __syncthreads();
  uint16_t* yt = reinterpret_cast<uint16_t*>(&stage[0]);
  const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 128 * wm + 32 * j + l32;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = 128 * wn + 32 * i + 8 * q + 4 * h;            // multiple of 4
        const int piece = (col >> 3) ^ (r & 7), half = (col >> 2) & 1;  // 16-byte piece, 8-byte half
        const f32x16_t& a = acc[i][j];
        *reinterpret_cast<uint2*>(yt + r * kMxTile + 8 * piece + 4 * half) =
            make_uint2(mx_bf16x2(a[4 * q], a[4 * q + 1]), mx_bf16x2(a[4 * q + 2], a[4 * q + 3]));
      }
  }
  __syncthreads();
  // 256 rows x 32 pieces of 16 bytes; thread t takes pieces t, t + 256, ...:
  // consecutive threads write consecutive pieces of a row.  Nontemporal: Y is
  // not read again by this kernel.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int64_t rows = p.m - m0 < kMxTile ? p.m - m0 : kMxTile;
  const int64_t cols = p.n - n0 < kMxTile ? p.n - n0 : kMxTile;
  const bool vec = (p.n & 7) == 0 && ((uintptr_t)p.y & 15) == 0;
#pragma unroll 4
  for (int pi = tid; pi < kMxTile * (kMxTile / 8); pi += 256) {
    const int r = pi >> 5, c8 = 8 * (pi & 31);
    if (r >= rows || c8 >= cols) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(yt + r * kMxTile + 8 * ((c8 >> 3) ^ (r & 7)));
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
                                                     reinterpret_cast<uint4*>(packed), scales);
}

void launch_mx_dequant(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, uint16_t* out,
                       hipStream_t s) {
  const int64_t pieces = rows * (k / 8);
  mx_dequant_kernel<<<mx_grid(pieces), 256, 0, s>>>(reinterpret_cast<const uint32_t*>(packed), scales, pieces,
                                                    reinterpret_cast<uint4*>(out));
}

bool mx_gemm_supported(int64_t m, int64_t n, int64_t k) {
  return m > 0 && n > 0 && k > 0 && k % kMxKC == 0 && m * (k / 2) < ((int64_t)1 << 32) &&
         n * (k / 2) < ((int64_t)1 << 32) && ((n + kMxTile - 1) / kMxTile) * ((m + kMxTile - 1) / kMxTile) < (1 << 30);
}

void launch_mx_gemm(const uint8_t* xq, const uint8_t* xs, int64_t m, const uint8_t* wq, const uint8_t* ws, int64_t n,
                    int64_t k, uint16_t* y, hipStream_t s) {
  const int64_t n_tiles = (n + kMxTile - 1) / kMxTile, m_tiles = (m + kMxTile - 1) / kMxTile;
  const MxArgs a{xq, xs, wq, ws, y, m, n, k, (int)n_tiles, (int)m_tiles};
  mx_gemm_kernel<<<dim3((unsigned)(n_tiles * m_tiles)), 256, 0, s>>>(a);
}

}  // namespace nvfp4
