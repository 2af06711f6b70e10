/*
 * nvfp4.h -- C ABI of libnvfp4.so, the MI355X (gfx950) NVFP4 weight-only linear.
 *
 * Format (homepage "Raphael Friedmann", NVFP4 bit diagram; imp
 * "docs/quantization.md", imp-quantize section; model card
 * "Qwen3.8-27B-NVFP4 (compressed-tensors)", "What is quantized"):
 *   - element: E2M1, 4 bits (sign, 2 exponent bits, 1 mantissa bit); magnitudes
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6;
 *   - two elements per byte ("packed nibbles"); element 2j in the low nibble of
 *     byte j, element 2j+1 in the high nibble;
 *   - one FP8 E4M3 (OCP E4M3FN) micro-scale per 16 consecutive K elements;
 *   - one FP32 tensor scale per tensor, stored as a multiplier;
 *   - weight-only: activations and outputs stay BF16 (W4A16).
 *
 * Shapes: a weight W is [n, k] row-major (n output features, k input
 * features), k a multiple of 16.  Its quantized form is
 *   packed  uint8 [n, k/2]     row-major,
 *   scales  uint8 [n, k/16]    row-major (E4M3 codes 0x00..0x7E),
 *   tscale  float [1].
 * Activations X are BF16 [m, k] row-major, outputs Y are BF16 [m, n]
 * row-major: Y = X . W_hat^T with W_hat = E2M1 * E4M3 * tscale.
 *
 * Conventions for every entry point:
 *   - Every pointer is a DEVICE pointer into caller-owned memory and must be
 *     16-byte aligned.  Nothing is allocated or freed by the library.
 *   - BF16 values are passed as uint16_t bit patterns; sizes are int64_t.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     stream-ordered and asynchronous: it never synchronises the device.
 *   - Arguments are validated on the host before any HIP call; a call that
 *     fails validation launches nothing.  NVFP4_ERR_DEVICE reports a HIP
 *     launch error (hipGetLastError) after launching.
 *   - Outputs must not overlap inputs (NVFP4_ERR_ALIAS).
 *   - Results are bitwise reproducible run to run (no floating-point atomics).
 *   - W and X must be finite; for non-finite inputs the outputs are unspecified
 *     but the call still terminates normally.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,       /* m < 0, n <= 0, k <= 0, k % 16 != 0, or a byte size overflows int64 */
  NVFP4_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  NVFP4_ERR_DEVICE = 4,      /* HIP reported an error (no device, launch failure) */
  NVFP4_ERR_UNSUPPORTED = 5, /* the current device is not gfx950, or an unknown kernel id */
  NVFP4_ERR_ALIAS = 6,       /* an output buffer overlaps an input buffer (appended after the five
                                codes above so that their values stay fixed) */
} nvfp4_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* nvfp4_status_string(int status);

/* Library version string, e.g. "nvfp4-mi355x 0.1.0". */
const char* nvfp4_version(void);

/*
 * Round-to-nearest BF16 -> NVFP4 quantizer (imp "docs/quantization.md",
 * imp-quantize section: uncalibrated round-to-nearest scales taken from the
 * block absmax).
 *   amax    = max |W|
 *   tscale  = fl32(amax / 2688)                                 (2688 = 6 * 448)
 *   scales  = per 16-element block, the E4M3 code nearest to 448 * bam / amax,
 *             bam = the block's max |w|; ties to the even code; 0 when bam = 0
 *   packed  = per element, sign = the BF16 sign bit, magnitude = the E2M1 code
 *             nearest to 2688 * |w| / (amax * s), s = the block scale value;
 *             ties to the even code, saturating at 6; 0 when s = 0
 * Every rounding decision is taken on the exact real quotient.
 * w: [n, k] BF16.  Outputs packed [n, k/2], scales [n, k/16], tscale [1].
 * Three kernels on the stream: per-workgroup maxima of |W| (held in packed
 * until the encode pass overwrites it), their reduction straight to tscale,
 * and the encode pass, which recovers amax from tscale exactly (the BF16 value
 * nearest to fl32(2688 * tscale) is amax for every finite BF16 amax).
 */
nvfp4_status nvfp4_quantize(const uint16_t* w, int64_t n, int64_t k,
                            uint8_t* packed, uint8_t* scales, float* tscale, void* stream);

/*
 * nvfp4_quantize in two launches instead of three, for a caller that has a
 * workspace: at least nvfp4_quantize_workspace_bytes() bytes (4096) of device
 * memory, 16-byte aligned, overlapping no argument; its contents before the
 * call do not matter and it is left holding partial maxima, so it must not be
 * a split-K workspace of the linear calls, whose counters must stay zero
 * (calls that overlap on one workspace race).  The amax pass
 * writes at most 1024 per-workgroup maxima of |W| to the workspace and every
 * workgroup of the encode pass reduces them itself (workgroup 0 also writes
 * tscale), so no reduction launch sits between the two.  The outputs are those
 * of nvfp4_quantize bit for bit.  A NULL or too small workspace runs
 * nvfp4_quantize.  Errors as nvfp4_quantize, plus NVFP4_ERR_SHAPE for a
 * negative workspace_bytes and NVFP4_ERR_ALIGN / NVFP4_ERR_ALIAS for the
 * workspace.
 */
int64_t nvfp4_quantize_workspace_bytes(void);
nvfp4_status nvfp4_quantize_ws(const uint16_t* w, int64_t n, int64_t k, uint8_t* packed, uint8_t* scales,
                               float* tscale, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Merged linears (model card "Qwen3.8-27B-NVFP4", "What is quantized": q/k/v
 * and gate/up members share one tensor scale; the amax spread inside a group
 * reaches 3.7x).  To quantize members held as separate tensors:
 *   1. set *amax = 0 (caller-owned device float),
 *   2. call nvfp4_amax_accumulate on every member (amax <- max(amax, max|W|)),
 *   3. call nvfp4_quantize_with_amax on every member with the same amax.
 * The outputs then equal, bit for bit, the rows of nvfp4_quantize applied to
 * the concatenated weight, and every member's tscale equals the shared one.
 * amax must hold a finite non-negative float; it must not overlap the outputs.
 */
nvfp4_status nvfp4_amax_accumulate(const uint16_t* w, int64_t n, int64_t k, float* amax, void* stream);

nvfp4_status nvfp4_quantize_with_amax(const uint16_t* w, int64_t n, int64_t k, const float* amax,
                                      uint8_t* packed, uint8_t* scales, float* tscale, void* stream);

/*
 * Dequantize to BF16: w_out = RNE_bf16( fl32( fl32(E2M1 * E4M3) * tscale ) ).
 * (The product of an E2M1 and an E4M3 value is exact in FP32.)
 * packed [n, k/2], scales [n, k/16], tscale [1] -> w_out [n, k] BF16.
 */
nvfp4_status nvfp4_dequant(const uint8_t* packed, const uint8_t* scales, const float* tscale,
                           int64_t n, int64_t k, uint16_t* w_out, void* stream);

/*
 * The W4A16 linear (model card "Qwen3.8-27B-NVFP4": weights NVFP4,
 * activations BF16; imp "docs/quantization.md", NVFP4 kernel pipeline: a
 * decode GEMV and a prefill GEMM):
 *   y[i, j] = RNE_bf16( tscale * sum_k x[i, k] * E2M1(w[j, k]) * E4M3(s[j, k/16]) )
 * accumulated in FP32.  The kernel is chosen from m: m = 1 -> GEMV,
 * 2 <= m <= 64 -> small-M MFMA kernel, m > 64 -> prefill MFMA GEMM.
 * x [m, k] BF16, packed [n, k/2], scales [n, k/16], tscale [1] -> y [m, n] BF16.
 * m = 0 is a no-op that returns NVFP4_OK once packed/scales/tscale/n/k are
 * valid; x and y may then be NULL.
 */
nvfp4_status nvfp4_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                          const uint8_t* packed, const uint8_t* scales, const float* tscale,
                          uint16_t* y, void* stream);

/*
 * The linear with a caller-provided workspace (same model card and page as
 * nvfp4_linear).  Two kernels can then split K across workgroups: the small-M
 * kernel (2 <= m <= 64) when its row blocks alone would not fill the device,
 * and the prefill GEMM when its 128 x 272 tiles would leave CUs idle (at most
 * 128 tiles, or up to 128 tiles past whole rounds of 256: those tiles only).
 * Each workgroup writes the FP32 partial sums of its K slice to the workspace,
 * and the last workgroup of each row block or tile to finish adds the slices
 * in slice order and writes y.  The result is therefore the same bits on every
 * run, but may differ in the last FP32 bits from nvfp4_linear's unsplit
 * summation.
 *
 * nvfp4_linear_workspace_bytes(m, n, k) returns the bytes this shape can use:
 * 0 when the chosen kernel needs none (m = 1, or no split), -1 for an invalid
 * shape.  It makes no HIP call.
 *
 * Workspace contract:
 *   - a device pointer, 16-byte aligned, not overlapping any argument buffer;
 *   - layout: the arrival counters in the first 16 KiB (the same bytes for
 *     every shape), then the FP32 partial sums;
 *   - zero-filled once before its first use; every call leaves the bytes that
 *     must start at zero (the arrival counters) at zero again, so later calls,
 *     of any shape, need no clearing;
 *   - calls that may run at the same time (other streams) need separate
 *     workspaces;
 *   - NULL, or workspace_bytes below the size returned above, runs the unsplit
 *     kernel (the result of nvfp4_linear) instead;
 *   - workspace_bytes < 0 is NVFP4_ERR_SHAPE.
 */
int64_t nvfp4_linear_workspace_bytes(int64_t m, int64_t n, int64_t k);

nvfp4_status nvfp4_linear_ws(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* packed, const uint8_t* scales, const float* tscale,
                             uint16_t* y, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * nvfp4_linear_ws without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The split-K
 * workspace is a library-owned device array of nvfp4_linear_noalloc_max_bytes()
 * bytes (8 MiB, enough for every split the small-M kernel plans), one copy per
 * GPU, held until the process ends; its address is looked up once per device,
 * on the first call with that device current, which also clears its counter
 * region with a kernel on `stream`.  No call allocates or frees memory.
 * Same arguments and errors as nvfp4_linear; results bit for bit those of
 * nvfp4_linear_ws with a workspace of at least nvfp4_linear_workspace_bytes(m,
 * n, k) bytes for m <= 64, and those of nvfp4_linear (unsplit) for the prefill
 * GEMM, whose split needs more than the array holds.  A shape whose workspace
 * would exceed the array returns NVFP4_ERR_SHAPE, and a failed address lookup
 * NVFP4_ERR_DEVICE.
 * Every call on one GPU shares that GPU's array and leaves its counters at
 * zero: calls that may overlap on one GPU (other streams, other threads)
 * race and must not be issued.
 */
int64_t nvfp4_linear_noalloc_max_bytes(void);
nvfp4_status nvfp4_linear_noalloc(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                  const uint8_t* packed, const uint8_t* scales, const float* tscale,
                                  uint16_t* y, void* stream);

/*
 * Kernel-native weight layout.  imp "docs/quantization.md", "NVFP4 kernel
 * pipeline" (Dense layers): the loader keeps the checkpoint's packed weights
 * and re-lays scale factors once for its prefill GEMM.  Here the same bytes
 * (values unchanged) are re-laid once, for k a multiple of 128, into the order
 * the gfx950 decode kernels read them:
 *   - rows in tiles of 16 (n padded with zero rows to a multiple of 16,
 *     tiles = ceil(n / 16)), k in quads of 128 elements; block (tile t,
 *     quad q) is 1152 bytes at offset (q * tiles + t) * 1152 (quad-major: the
 *     blocks of consecutive tiles for one quad lie side by side);
 *   - its first 1024 bytes are 64 slots of 16 bytes: slot 16 g + r (g = 0..3,
 *     r = 0..15) holds, as 4-byte words i = 0..3, the elements
 *     128 q + 32 i + 8 g .. + 8 of row 16 t + r (low nibble first, as in
 *     packed);
 *   - its last 128 bytes are 32 words: word 16 h + r (h = 0, 1) holds, as
 *     byte i, the E4M3 scale of block 8 q + 2 i + h of row 16 t + r.
 * A wavefront then loads the weights of one (tile, quad) as one contiguous
 * kilobyte and their scales as one 128-byte line, and the tiles a workgroup
 * reads for one quad are one contiguous run.  The tensor scale is unchanged
 * and passed separately.
 *
 * nvfp4_prepared_bytes(n, k): size of the layout, -1 when n <= 0, k <= 0,
 * k % 128 != 0 or the size overflows (no HIP call).
 * nvfp4_prepare: packed [n, k/2] + scales [n, k/16] -> prepared (16-byte
 * aligned, nvfp4_prepared_bytes(n, k) bytes, overlapping neither input).
 * nvfp4_dequant_prepared: prepared + tscale -> w_out [n, k] BF16, bit for bit
 * the nvfp4_dequant of the weight it was prepared from.
 * nvfp4_linear_prepared: y [m, n] = x [m, k] . W_hat^T from the prepared
 * weight, for 1 <= m <= 32 (the decode and batched-decode shapes; larger m is
 * NVFP4_ERR_UNSUPPORTED: the prefill GEMM reads the checkpoint layout); m = 0
 * is a no-op.  m = 1 runs a GEMV on the vector ALU (no workspace); 2 <= m
 * <= 32 the matrix-core kernel.  Accumulation in FP32 in a different order
 * than nvfp4_linear, so within the same tolerance, not bit-identical to it.
 * Workspace: as for nvfp4_linear_ws, with
 * nvfp4_linear_prepared_workspace_bytes(m, n, k) bytes (0: none needed; NULL
 * or too small runs without a K split).
 * Errors as nvfp4_linear; a k that is not a multiple of 128 is NVFP4_ERR_SHAPE.
 */
int64_t nvfp4_prepared_bytes(int64_t n, int64_t k);
nvfp4_status nvfp4_prepare(const uint8_t* packed, const uint8_t* scales, int64_t n, int64_t k, uint8_t* prepared,
                           void* stream);
nvfp4_status nvfp4_dequant_prepared(const uint8_t* prepared, const float* tscale, int64_t n, int64_t k,
                                    uint16_t* w_out, void* stream);
int64_t nvfp4_linear_prepared_workspace_bytes(int64_t m, int64_t n, int64_t k);
nvfp4_status nvfp4_linear_prepared(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* prepared,
                                   const float* tscale, uint16_t* y, void* workspace, int64_t workspace_bytes,
                                   void* stream);

/*
 * Measurement aid (not a step of the linear): reads `bytes` bytes (a positive
 * multiple of 16) of device memory at `src` once, with 16-byte loads, in
 * nvfp4_stream_read_sink_words(bytes) <= 8192 workgroups; workgroup b stores
 * the XOR of the 32-bit words it read to sink[b] (caller-owned device memory
 * of that many words, 4-byte aligned, not overlapping src), so the XOR of
 * those words is the XOR of the whole buffer.  Its rate is the plain HBM read
 * rate on the device, against which the streaming kernels above are measured.
 * src 16-byte aligned.  nvfp4_stream_read_sink_words returns -1 for a bad size.
 */
int64_t nvfp4_stream_read_sink_words(int64_t bytes);
nvfp4_status nvfp4_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Kernel ids for nvfp4_linear_forced. */
#define NVFP4_KERNEL_AUTO 0
#define NVFP4_KERNEL_GEMV 1     /* VALU dot-product GEMV; any m (rows handled independently) */
#define NVFP4_KERNEL_SMALL_M 2  /* MFMA kernel with 16/32-row X tiles; any m */
#define NVFP4_KERNEL_PREFILL 3  /* MFMA GEMM with large tiles; any m */

/*
 * Same as nvfp4_linear but runs the named kernel for any m (used by tests to
 * cross-check the kernels against each other and against the oracle).
 * An unknown kernel id returns NVFP4_ERR_UNSUPPORTED.
 */
nvfp4_status nvfp4_linear_forced(int kernel_id, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                 const uint8_t* packed, const uint8_t* scales, const float* tscale,
                                 uint16_t* y, void* stream);

/*
 * Expert stacks (mixture-of-experts layers).  imp "docs/quantization.md": in
 * the NVFP4 kernel pipeline, a MoE layer's per-expert weights become one
 * contiguous [ne, N, K_packed] buffer per layer and projection, and the
 * imp-quantize section notes that 3-D expert stacks need a per-expert path.
 * Each expert is its own quantized tensor with its own tensor scale:
 *   w [e, n, k] BF16 -> packed [e, n, k/2], scales [e, n, k/16], tscale [e]
 * where matrix i of the outputs equals nvfp4_quantize applied to w[i], bit
 * for bit.  e = 0 is a no-op.  The same scratch use as nvfp4_quantize:
 * tscale[i] is written first and its packed matrix holds per-workgroup
 * maxima until the last kernels overwrite them.
 */
nvfp4_status nvfp4_quantize_experts(const uint16_t* w, int64_t e, int64_t n, int64_t k,
                                    uint8_t* packed, uint8_t* scales, float* tscale, void* stream);

/* Dequantize an expert stack: w_out[i] = nvfp4_dequant of matrix i (same
 * layouts as nvfp4_quantize_experts; w_out [e, n, k] BF16). */
nvfp4_status nvfp4_dequant_experts(const uint8_t* packed, const uint8_t* scales, const float* tscale,
                                   int64_t e, int64_t n, int64_t k, uint16_t* w_out, void* stream);

/*
 * Routed W4A16 linear over an expert stack (the decode path of a MoE layer
 * with top-k routing; same stack layout as above):
 *   y[t, j, :] = nvfp4_linear(x[t, :], matrix route[t, j] of the stack)
 * for t < t_count, j < topk.  x [t_count, k] BF16, route [t_count, topk]
 * int32 expert ids (device memory), packed [e, n, k/2], scales [e, n, k/16],
 * tscale [e] -> y [t_count, topk, n] BF16.  Each (t, j) pair runs the GEMV
 * on its expert's matrix (for k a multiple of 512 up to 5120 the same kernel,
 * hence the same bits, as nvfp4_linear with m = 1).  Combining the topk
 * outputs with the router's weights is the caller's.
 * An expert id outside [0, e) gives a row of zeros for that pair (ids are
 * device data, so they are checked on the device, not reported).
 * t_count = 0 is a no-op; topk >= 1 and e >= 1 are required; route must be
 * 4-byte aligned and the other pointers 16-byte aligned; y must not overlap
 * an input.
 */
nvfp4_status nvfp4_linear_routed(const uint16_t* x, int64_t t_count, int64_t topk, const int32_t* route,
                                 int64_t e, int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                                 const float* tscale, uint16_t* y, void* stream);

/*
 * Grouped W4A16 linear over an expert stack: the prefill path of a MoE layer
 * (many tokens, top-k routing).  Same arguments, layouts and result as
 * nvfp4_linear_routed (y [t_count, topk, n]; within the linear's tolerance,
 * since a different kernel sums in a different order; an expert id outside
 * [0, e) gives a row of zeros), plus a caller-owned device workspace of at
 * least nvfp4_linear_grouped_workspace_bytes(t_count, topk, e) bytes,
 * 16-byte aligned, overlapping no argument.  On the stream, one workgroup
 * counts and sorts the (t, j) pairs by expert into the workspace, then one
 * GEMM launch multiplies each expert's matrix with its pairs' activation rows
 * in 128-row tiles (and zeroes the rows of out-of-range ids), so an expert's
 * weights are read once per 272 output columns however many tokens chose it
 * (the routed GEMV reads them once per pair).  The order
 * of pairs within an expert is not deterministic; the output is, bit for bit.
 * Where the GEMM's limits are not met (k not a multiple of 256, t_count * k
 * above 2^31, or 32-bit pair and tile counts exceeded) the call runs
 * nvfp4_linear_routed's GEMV instead and leaves the workspace unused.
 * Errors: as nvfp4_linear_routed; a NULL workspace (t_count > 0) is
 * NVFP4_ERR_NULL, a workspace_bytes below the size above NVFP4_ERR_SHAPE.
 * The workspace must not be shared by calls in flight at the same time.
 */
int64_t nvfp4_linear_grouped_workspace_bytes(int64_t t_count, int64_t topk, int64_t e);

nvfp4_status nvfp4_linear_grouped(const uint16_t* x, int64_t t_count, int64_t topk, const int32_t* route,
                                  int64_t e, int64_t n, int64_t k, const uint8_t* packed,
                                  const uint8_t* scales, const float* tscale, uint16_t* y, void* workspace,
                                  int64_t workspace_bytes, void* stream);

/*
 * Paged FP4 KV-cache gather.  imp "docs/quantization.md", KV-cache
 * paragraphs: an NVFP4 KV cache keeps E2M1 values with UE4M3 micro-scales and
 * an MXFP4 KV cache the same nibbles with UE8M0 micro-scales per 32 elements;
 * for chunked prefill the past chunks' K/V are gathered from the paged cache
 * into FP16 and joined with the current chunk before attention.
 *
 * One cache (one layer's K or V) in pages of block_size tokens:
 *   codes  [num_blocks, block_size, heads, head_dim / 2] uint8, element 2j in
 *          the low nibble of byte j;
 *   scales [num_blocks, block_size, heads, head_dim / G] uint8: G = 16, E4M3
 *          (format NVFP4_KV_NVFP4, with one FP32 tensor scale *tscale), or
 *          G = 32, UE8M0 = 2^(byte - 127), 0xFF NaN (NVFP4_KV_MXFP4, no tensor
 *          scale: tscale is ignored and may be NULL).
 * For sequence s < seqs and token i < min(seq_lens[s], max_blocks * block_size):
 *   out[dst_start[s] + i, :, :] = decode(page block_table[s, i / block_size],
 *                                        slot i % block_size)
 * with decode = RNE_out(fl32(fl32(E2M1 * E4M3) * tscale)) (NVFP4) or
 * RNE_out(E2M1 * 2^(byte - 127)) (MXFP4), out [out_rows, heads, head_dim]
 * FP16 (NVFP4_OUT_F16) or BF16 (NVFP4_OUT_BF16).  block_table [seqs,
 * max_blocks], seq_lens [seqs] and dst_start [seqs] are int32 device data, so
 * they are not validated on the host: a page id outside [0, num_blocks) gives
 * zero rows, a negative length gathers nothing, and output rows outside
 * [0, out_rows) are skipped.  Every other output row keeps its contents (the
 * caller writes the current chunk's K/V around the gathered rows).
 * Errors: an unknown format or out_type is NVFP4_ERR_UNSUPPORTED;
 * head_dim % G != 0, non-positive num_blocks, block_size, heads, head_dim or
 * max_blocks, negative seqs or out_rows, seqs * max_blocks > 2^31 - 1 or a
 * byte size overflow is NVFP4_ERR_SHAPE; codes and out must be 16-byte
 * aligned, tscale and the int32 arrays 4-byte aligned; out must not overlap
 * an input.  seqs = 0 is a no-op.
 */
#define NVFP4_KV_NVFP4 0
#define NVFP4_KV_MXFP4 1
#define NVFP4_OUT_F16 0
#define NVFP4_OUT_BF16 1

nvfp4_status nvfp4_kv_gather(int format, int out_type, const uint8_t* codes, const uint8_t* scales,
                             const float* tscale, int64_t num_blocks, int64_t block_size, int64_t heads,
                             int64_t head_dim, const int32_t* block_table, int64_t max_blocks,
                             const int32_t* seq_lens, const int32_t* dst_start, int64_t seqs, uint16_t* out,
                             int64_t out_rows, void* stream);

/*
 * MXFP4 tensors and the W4A4 (FP4 x FP4) linear.  imp "docs/quantization.md",
 * MXFP4 paragraph: the NVFP4 E2M1 nibble layout with a UE8M0 micro-scale per 32
 * elements and no separate tensor scale, the format FP4 matrix cores take
 * natively (an MXFP4 prefill runs at full FP4 rate); round-to-nearest MXFP4 is
 * the page's quantizer.  Layout of a rows x k tensor (k a multiple of 32):
 * packed [rows, k/2] (element 2j in the low nibble of byte j) and scales
 * [rows, k/32], scale byte e meaning 2^(e - 127) (0xFF NaN).
 *
 * nvfp4_mx_quantize: BF16 [rows, k] -> MXFP4, round to nearest with the OCP
 * MX shared scale: per block of 32, e = clamp(floor(log2(amax)) - 2 + 127, 0,
 * 254) (0 for an all-zero block), code = sign | the E2M1 magnitude nearest to
 * |v| / 2^(e - 127), ties to the even code, saturating at 6.  Bit for bit the
 * same for weights and activations.  rows = 0 is a no-op.
 * nvfp4_mx_dequant: MXFP4 -> BF16 [rows, k] (E2M1 * 2^(e - 127), RNE).
 * nvfp4_mx_gemm: y [m, n] BF16 = xq [m, k] . wq [n, k]^T on the FP4 matrix
 * cores (FP32 accumulation), from already quantized operands.
 * nvfp4_mx_linear_w4a4: the same with x [m, k] BF16, quantized on the stream
 * into a caller-owned workspace of nvfp4_mx_linear_w4a4_workspace_bytes(m, k)
 * bytes (16-byte aligned, overlapping no argument) and then multiplied.
 * Results are within 2e-3 of sum_k |xq * wq| of the exact product of the
 * quantized operands, plus the BF16 output rounding.
 * Errors: k % 32 != 0, n <= 0 or a size overflow is NVFP4_ERR_SHAPE (also a
 * workspace below the size above); the GEMM needs k % 128 == 0 and
 * m * k / 2, n * k / 2 < 2^32, else NVFP4_ERR_UNSUPPORTED; every pointer
 * 16-byte aligned; outputs must not overlap inputs; m = 0 is a no-op.
 */
nvfp4_status nvfp4_mx_quantize(const uint16_t* w, int64_t rows, int64_t k, uint8_t* packed, uint8_t* scales,
                               void* stream);
nvfp4_status nvfp4_mx_dequant(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t k,
                              uint16_t* out, void* stream);
nvfp4_status nvfp4_mx_gemm(const uint8_t* xq, const uint8_t* xs, int64_t m, const uint8_t* wq, const uint8_t* ws,
                           int64_t n, int64_t k, uint16_t* y, void* stream);
int64_t nvfp4_mx_linear_w4a4_workspace_bytes(int64_t m, int64_t k);
nvfp4_status nvfp4_mx_linear_w4a4(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* wq,
                                  const uint8_t* ws, uint16_t* y, void* workspace, int64_t workspace_bytes,
                                  void* stream);

/*
 * NVFP4 x NVFP4 linear (activations quantized too).  imp "docs/quantization.md",
 * the Modelopt row of the loader table: an NVFP4 x NVFP4 prefill beside the
 * weight-only path.  Each call quantizes x [m, k] BF16 to NVFP4 exactly as
 * nvfp4_quantize quantizes a weight (one tensor scale from max |x| over the
 * call, an E4M3 scale per 16 along k, E2M1 codes), then
 *   y [m, n] BF16 = x_hat . w_hat^T,
 * with FP32 accumulation.  The FP4 matrix cores of gfx950 take one power-of-two
 * scale per 32 elements, not an E4M3 scale per 16, so the product runs on the
 * BF16 matrix cores: each x_hat element without its tensor scale (E2M1 * E4M3,
 * at most 6 significant bits) is exact in BF16, and the two tensor scales are
 * applied once, as fl32(ts_w * ts_x), to the FP32 sums.  Results are within
 * 2e-3 of sum_k |x_hat * w_hat| of the exact product, plus the BF16 output
 * rounding.
 *
 * Workspace: nvfp4_linear_w4a4_workspace_bytes(m, k) bytes of device memory,
 * 16-byte aligned, overlapping no argument, no clearing needed; -1 for an
 * invalid shape, 0 for m = 0.  After the call it holds, each part starting on
 * a 16-byte boundary: x's codes [m, k/2], x's E4M3 scales [m, k/16], the floats
 * {ts_y, max |x|, ts_x, unused}, and x_hat / ts_x as BF16 [m, k].
 * Errors: those of nvfp4_linear; a NULL workspace (m > 0) is NVFP4_ERR_NULL, a
 * workspace below the size above NVFP4_ERR_SHAPE.  Concurrent calls need
 * separate workspaces.
 */
int64_t nvfp4_linear_w4a4_workspace_bytes(int64_t m, int64_t k);
nvfp4_status nvfp4_linear_w4a4(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                               const uint8_t* scales, const float* tscale, uint16_t* y, void* workspace,
                               int64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
