// Internal launchers of the gfx950 kernels (host side).  Callers validate every
// argument first; the launchers assume valid shapes and aligned pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Quantizer and dequantizer over a stack of `count` matrices of n_elems
// elements each, stored back to back (count = 1 for one matrix); amax and
// tscale hold one value per matrix.
void launch_amax(const uint16_t* w, int64_t n_elems, float* amax, hipStream_t s);
// *amax = max |w|, with per-workgroup maxima in part (at least n_elems / 8 32-bit words).
void launch_amax_set(const uint16_t* w, int64_t n_elems, uint32_t* part, float* amax, hipStream_t s);
// amax[i] = max |w_i|, with matrix i's per-workgroup maxima at part + i * n_elems / 8.
void launch_amax_set_stack(const uint16_t* w, int64_t count, int64_t n_elems, uint32_t* part, float* amax,
                           hipStream_t s);
void launch_finalize_tscale(const float* amax, float* tscale, int64_t count, hipStream_t s);
// tscale[i] = fl32(max |w_i| / 2688) (partial maxima in part as for launch_amax_set_stack), and the
// quantize pass that recovers amax from it: the quantizer in three launches.
void launch_tscale_set_stack(const uint16_t* w, int64_t count, int64_t n_elems, uint32_t* part, float* tscale,
                             hipStream_t s);
void launch_quantize_from_tscale(const uint16_t* w, int64_t count, int64_t n_elems, const float* tscale,
                                 uint8_t* packed, uint8_t* scales, hipStream_t s);
// Two launches: at most 1024 per-workgroup maxima of |w| into parts (4 KiB),
// then the encode pass, each of whose workgroups reduces them; workgroup 0
// writes tscale = fl32(amax / 2688).
void launch_quantize_shared_amax(const uint16_t* w, int64_t n_elems, uint32_t* parts, float* tscale,
                                 uint8_t* packed, uint8_t* scales, hipStream_t s);
void launch_quantize(const uint16_t* w, int64_t count, int64_t n_elems, const float* amax, uint8_t* packed,
                     uint8_t* scales, hipStream_t s);
void launch_dequant(const uint8_t* packed, const uint8_t* scales, const float* tscale, int64_t count, int64_t n_elems,
                    uint16_t* out, hipStream_t s);
// launch_quantize of one matrix that also writes, per element, the exact BF16
// value E2M1 * E4M3 (the tensor scale left out) to decoded [n_elems], and the
// scalars ts_x = fl32(amax / 2688), ts_y = fl32(ts_w * ts_x) (NVFP4 x NVFP4).
void launch_quantize_decode(const uint16_t* w, int64_t n_elems, const float* amax, uint8_t* packed, uint8_t* scales,
                            uint16_t* decoded, const float* ts_w, float* ts_x, float* ts_y, hipStream_t s);

void launch_gemv(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                 const float* tscale, uint16_t* y, hipStream_t s);
// Routed GEMV over an expert stack: for pair p = t * topk + j (p < t_count * topk),
// y[p, :] = x[t, :] . W_e^T with e = route[p]; W_e is matrix e of the stack
// (packed + e n k / 2, scales + e n k / 16, tscale[e]).  Pairs whose expert id
// is outside [0, experts) get zeros.
void launch_gemv_routed(const uint16_t* x, int64_t t_count, int64_t topk, const int32_t* route, int64_t experts,
                        int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales, const float* tscale,
                        uint16_t* y, hipStream_t s);
// Small-M kernel.  With a workspace of at least skinny_workspace_bytes(m, n, k)
// bytes (zero-filled before its first use; left that way by every launch) it may
// split K across workgroups; with none it runs unsplit.
// The workspace starts with kSkinnyCounterBytes of arrival counters (the same
// region for every shape), followed by the FP32 partial sums.
constexpr int64_t kSkinnyCounterBytes = 16384;
int64_t skinny_workspace_bytes(int64_t m, int64_t n, int64_t k);
void launch_skinny(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                   const float* tscale, uint16_t* y, void* workspace, int64_t workspace_bytes, hipStream_t s);
// The kernel-native weight layout (16-row tiles x 128-element quads, 1152
// bytes per (tile, quad); k a multiple of 128): its size, the conversion from
// the checkpoint layout, and its dequantizer.
int64_t prepared_bytes(int64_t n, int64_t k);
void launch_prepare(const uint8_t* packed, const uint8_t* scales, int64_t n, int64_t k, uint8_t* out, hipStream_t s);
void launch_dequant_prepared(const uint8_t* prep, const float* tscale, int64_t n, int64_t k, uint16_t* out,
                             hipStream_t s);
// Small-M MFMA kernel on the kernel-native layout, 1 <= m <= 32.  With a plan
// that splits K (slices > 1) it needs a workspace of plan.ws_bytes laid out as
// for launch_skinny.
struct SmallMPlan {
  int rows = 16, tiles = 1, slices = 1, quads = 1;
  int64_t row_blocks = 1, npad = 0, ws_bytes = 0;
};
bool small_m_supported(int64_t m, int64_t n, int64_t k);
SmallMPlan small_m_plan(int64_t m, int64_t n, int64_t k, bool split);
// M = 1 on the kernel-native layout (k a multiple of 128).
void launch_gemv_prepared(const uint16_t* x, int64_t n, int64_t k, const uint8_t* prep, const float* tscale,
                          uint16_t* y, hipStream_t s);
void launch_small_m(const SmallMPlan& pl, const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* prep,
                    const float* tscale, uint16_t* y, void* workspace, hipStream_t s);
// Prefill GEMM.  With a workspace of at least prefill_workspace_bytes(m, n, k)
// bytes (zero-filled before its first use; left that way by every launch), a
// tile count that leaves CUs idle splits some tiles along K (prefill_split);
// with none it runs one tile per workgroup.  The workspace starts with
// kSkinnyCounterBytes of arrival counters, then the FP32 partial tiles.
void launch_gemm_prefill(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                         const uint8_t* scales, const float* tscale, uint16_t* y, void* workspace,
                         int64_t workspace_bytes, hipStream_t s);
// Streaming prefill GEMM (K a multiple of 256); launch_gemm_prefill uses it when supported.
bool prefill_dma_supported(int64_t m, int64_t n, int64_t k);
struct PdSplit {
  int dp = 0;    // whole tiles, one workgroup each, launched first
  int tail = 0;  // tiles after them, each split along K
  int c = 0;     // slices per split tile (0: no split)
};
PdSplit prefill_split(int64_t m, int64_t n, int64_t k);
int64_t prefill_workspace_bytes(int64_t m, int64_t n, int64_t k);
void launch_prefill_dma(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                        const uint8_t* scales, const float* tscale, uint16_t* y, void* workspace,
                        int64_t workspace_bytes, hipStream_t s);

// Grouped prefill over an expert stack (K a multiple of 256, t_count * k <= 2^31,
// int32 pair indices and workgroup ids):
// the pairs of the top-k routing sorted by expert in a workspace of
// grouped_workspace_bytes(pairs, experts) bytes, then the prefill GEMM per
// expert tile.  Same result as launch_gemv_routed (within the linear's
// tolerance), including zero rows for out-of-range expert ids.
bool prefill_grouped_supported(int64_t t_count, int64_t topk, int64_t experts, int64_t n, int64_t k);
int64_t prefill_grouped_tile_bound(int64_t pairs, int64_t experts);
int64_t grouped_workspace_bytes(int64_t pairs, int64_t experts);
void launch_prefill_grouped(const uint16_t* x, int64_t topk, const int32_t* groups, int64_t pairs, int64_t experts,
                            int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales, const float* tscale,
                            uint16_t* y, hipStream_t s);
void launch_linear_grouped(const uint16_t* x, int64_t t_count, int64_t topk, const int32_t* route, int64_t experts,
                           int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales, const float* tscale,
                           uint16_t* y, void* workspace, hipStream_t s);

// Paged FP4 KV-cache gather (mx: UE8M0 scales per 32, else E4M3 per 16 and
// one FP32 tensor scale; bf16: BF16 output, else FP16).  row_elems = heads *
// head_dim, a multiple of 16 (32 when mx).  One workgroup per (sequence, block
// table entry): seqs * max_blocks < 2^31.
void launch_kv_gather(bool mx, bool bf16, const uint8_t* codes, const uint8_t* scales, const float* tscale,
                      int64_t num_blocks, int64_t block_size, int64_t row_elems, const int32_t* block_table,
                      int64_t max_blocks, const int32_t* seq_lens, const int32_t* dst_start, int64_t seqs,
                      uint16_t* out, int64_t out_rows, hipStream_t s);

// MXFP4 (UE8M0 scale per 32, no tensor scale).  Quantizer and dequantizer
// over rows x k (k a multiple of 32); W4A4 GEMM y [m, n] = xq . wq^T for k a
// multiple of 128 and m * k / 2, n * k / 2 < 2^32 (mx_gemm_supported).
void launch_mx_quantize(const uint16_t* w, int64_t rows, int64_t k, uint8_t* packed, uint8_t* scales, hipStream_t s);
void launch_mx_dequant(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, uint16_t* out,
                       hipStream_t s);
bool mx_gemm_supported(int64_t m, int64_t n, int64_t k);
void launch_mx_gemm(const uint8_t* xq, const uint8_t* xs, int64_t m, const uint8_t* wq, const uint8_t* ws, int64_t n,
                    int64_t k, uint16_t* y, hipStream_t s);

// Plain streaming read of `bytes` bytes (a multiple of 16) of device memory by
// stream_read_blocks(bytes) <= kStreamSinkWords workgroups; workgroup b stores the
// XOR of the 32-bit words it read to sink[b].
constexpr int64_t kStreamSinkWords = 8192;
int64_t stream_read_blocks(int64_t bytes);
void launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace nvfp4
