"""CPU oracle for the FP4 KV-cache gather.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code, table or helper with the HIP path.

Sources (web pages, cited by title and section):
  * imp "docs/quantization.md", KV-cache paragraphs: an NVFP4 KV cache
    stores E2M1 values with UE4M3 micro-scales, an MXFP4 KV cache the same
    E2M1 nibbles with UE8M0 micro-scales; both hold K/V at a quarter of FP16.
    For chunked prefill, the past chunks' K/V are gathered from the paged
    cache into FP16 (an E2M1 -> FP16 conversion with the micro-scale folded
    in) and joined with the current chunk before attention.
  * same page, the MXFP4 paragraph: the same E2M1 nibble layout as NVFP4,
    a UE8M0 micro-scale per 32 elements, no separate tensor scale.
  * The E2M1 and E4M3 tables are those of nvfp4_oracle (pinned there); UE8M0
    is the OCP Microscaling format's scale byte (2^(e - 127), 0xFF NaN): the
    pages name the format but do not define it.

Readings taken where the pages are silent or open:
  R14 cache layout  one cache per layer and per K or V, in fixed-size pages ("blocks") of block_size
                    tokens: codes [num_blocks, block_size, heads, head_dim / 2] (element 2j in the low
                    nibble of byte j, as for weights), scales [num_blocks, block_size, heads,
                    head_dim / G] with G = 16 (NVFP4, E4M3) or 32 (MXFP4, UE8M0), blocks running
                    along head_dim.  An NVFP4 cache has one FP32 tensor scale, like NVFP4 weights;
                    an MXFP4 cache has none.
  R15 decode        NVFP4: out = RNE_out(fl32(fl32(E2M1 * E4M3) * tscale)), the weights' dequant with
                    FP16 or BF16 as the output type; MXFP4: out = RNE_out(E2M1 * 2^(e - 127)) (one
                    rounding; a product beyond FP32's range overflows to infinity like the output
                    types), scale byte 0xFF gives NaN.
  R16 gather        for sequence s and its token i < min(seq_lens[s], max_blocks * block_size):
                    out[dst_start[s] + i] = decode(page block_table[s, i // block_size], slot
                    i % block_size), a [heads, head_dim] row.  A page id outside [0, num_blocks) gives a
                    zero row; output rows outside [0, out_rows) are not written; every other output row
                    keeps its contents (the caller places the current chunk around the gathered rows).

Parity pins: tests/test_oracle_pins.py checks the UE8M0 table against
torch's float8_e8m0fnu, the decode against exact-rational products rounded
by numpy's and torch's casts, and the gather's indexing by brute force on
pages whose values name their source.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from oracle.nvfp4_oracle import E2M1_TABLE, E4M3_TABLE, f32_to_bf16_rne, unpack_nibbles

NVFP4, MXFP4 = "nvfp4", "mxfp4"
F16, BF16 = "f16", "bf16"
GROUP = {NVFP4: 16, MXFP4: 32}


def _ue8m0_from_bits(code: int) -> float:
    """OCP MX scale byte: 2^(code - 127), 0xFF NaN."""
    return float("nan") if code == 0xFF else float(np.ldexp(1.0, code - 127))


UE8M0_TABLE = np.array([_ue8m0_from_bits(c) for c in range(256)], dtype=np.float64)


def decode_values(fmt: str, codes: np.ndarray, scales: np.ndarray, tscale=None) -> np.ndarray:
    """R15 before the output rounding: codes [..., D/2] uint8, scales [..., D/G] uint8 -> values [..., D].

    NVFP4: float32 fl32(E2M1 * E4M3) * fl32(tscale) rounded to float32 (the product E2M1 * E4M3 has at
    most 6 significant bits and is exact in float32).  MXFP4: the exact float64 product E2M1 * 2^(e-127)
    (at most 2 significant bits; float64 holds it for every e).
    """
    g = GROUP[fmt]
    codes = np.asarray(codes, dtype=np.uint8)
    lead, half = codes.shape[:-1], codes.shape[-1]
    e2m1 = E2M1_TABLE[unpack_nibbles(codes.reshape(-1, half))].reshape(lead + (2 * half,))
    if fmt == NVFP4:
        sc = np.repeat(E4M3_TABLE[np.asarray(scales, dtype=np.uint8)], g, axis=-1)
        prod = (e2m1 * sc).astype(np.float32)
        assert np.array_equal(prod.astype(np.float64), e2m1 * sc, equal_nan=True)
        with np.errstate(over="ignore", invalid="ignore"):
            return prod * np.float32(tscale)
    sc = np.repeat(UE8M0_TABLE[np.asarray(scales, dtype=np.uint8)], g, axis=-1)
    with np.errstate(invalid="ignore"):
        return e2m1 * sc


def round_out(values: np.ndarray, out: str) -> np.ndarray:
    """R15's final rounding: float32 / float64 values -> FP16 or BF16 bits (uint16), nearest even.

    FP16 through numpy's cast (correctly rounded from either width); BF16 from float32 through torch's
    cast, and from float64 (MXFP4 products) after an exact float64 -> float32 step where the value is
    representable in float32 (2 significant bits always are; beyond float32's range the value overflows
    to infinity exactly as BF16 would, and below its subnormals it rounds to zero in both).
    """
    v = np.asarray(values)
    if out == F16:
        with np.errstate(over="ignore"):
            return v.astype(np.float16).view(np.uint16)
    with np.errstate(over="ignore", under="ignore"):
        v32 = v.astype(np.float32)
    return f32_to_bf16_rne(v32)


def decode_rows(fmt: str, out: str, codes: np.ndarray, scales: np.ndarray, tscale=None) -> np.ndarray:
    """R15: cache rows -> output bits."""
    return round_out(decode_values(fmt, codes, scales, tscale), out)


def kv_gather_ref(fmt: str, out: str, codes: np.ndarray, scales: np.ndarray, tscale, block_table: np.ndarray,
                  seq_lens: np.ndarray, dst_start: np.ndarray, out_init: np.ndarray) -> np.ndarray:
    """R16: the gathered output [out_rows, heads, head_dim] (uint16 bits), starting from out_init.

    codes [num_blocks, block_size, heads, head_dim/2], scales [num_blocks, block_size, heads, head_dim/G],
    block_table [seqs, max_blocks] int, seq_lens [seqs] int, dst_start [seqs] int.
    """
    nb, bs, heads, half = codes.shape
    y = np.array(out_init, dtype=np.uint16, copy=True)
    out_rows = y.shape[0]
    max_blocks = block_table.shape[1]
    for s in range(block_table.shape[0]):
        n = min(max(int(seq_lens[s]), 0), max_blocks * bs)
        for i in range(n):
            row = int(dst_start[s]) + i
            if row < 0 or row >= out_rows:
                continue
            page = int(block_table[s, i // bs])
            if page < 0 or page >= nb:
                y[row] = 0
            else:
                y[row] = decode_rows(fmt, out, codes[page, i % bs], scales[page, i % bs], tscale)
    return y
