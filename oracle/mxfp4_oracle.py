"""CPU oracle for MXFP4 tensors and the W4A4 (FP4 x FP4) linear.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code, table or helper with the HIP path.

Sources (web pages, cited by title and section):
  * imp "docs/quantization.md", MXFP4 paragraph: the same FP4 E2M1 nibble
    layout as NVFP4, a UE8M0 micro-scale per 32 elements and no separate
    tensor scale: the format the FP4 tensor cores take natively, so an MXFP4
    prefill runs at full FP4 throughput; the format table lists MXFP4 weights
    at 4.5 bits per element; the quality paragraph quantizes MXFP4 by round to
    nearest.
  * same page, the note on Modelopt checkpoints: an NVFP4 x NVFP4 prefill
    (activations quantized too) exists beside the weight-only path.
  * The E2M1 table is nvfp4_oracle's and UE8M0 is kv_oracle's (both pinned).
    How a block's shared scale is chosen is not on the pages; the OCP
    Microscaling format's conversion is the plain reading (R17).

Readings taken where the pages are silent or open:
  R17 MXFP4 quantizer  per block of 32 consecutive elements along K: amax = max |v|;
                       scale byte E = clamp(floor(log2(amax)) - 2 + 127, 0, 254) (2 = the exponent of
                       E2M1's largest value 6 = 1.5 * 2^2), E = 0 when amax = 0; element code = sign bit |
                       the E2M1 magnitude nearest to the real |v| / 2^(E - 127), ties to the even code,
                       saturating at 6.  amax / 2^(E - 127) lies in [4, 8), so the block maximum maps to 4
                       or 6 and values above 6 * 2^(E-127) clip to 6.
  R18 layouts          packed [R, K/2] (element 2j in the low nibble of byte j), scales [R, K/32]
                       UE8M0, row-major; the same for weights [N, K] and activations [M, K].
  R19 W4A4 linear      Y[m, n] = sum_k Xq[m, k] * Wq[n, k], Xq and Wq the MXFP4 values of R17 (X quantized
                       the same way as W, per 32 along K); accepted within 2e-3 * sum_k |Xq * Wq| plus the
                       BF16 output rounding (R11's form).

Parity pins: tests/test_oracle_pins.py checks the quantizer against an
exhaustive nearest-value search over exact rationals, the block-maximum and
saturation closed forms and idempotence, and the linear against exact
rational sums and one-hot closed forms.  No function here is "parity unpinned".
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from oracle.kv_oracle import UE8M0_TABLE
from oracle.nvfp4_oracle import (E2M1_TABLE, _E2M1_MIDS, _nearest_code_ties_even, bf16_to_f64, linear_violations,
                                 pack_nibbles, unpack_nibbles)

MX_BLOCK = 32
E2M1_EMAX = 2              # 6 = 1.5 * 2^2


def block_scale_bytes(w_bits: np.ndarray) -> np.ndarray:
    """R17: BF16 [R, K] -> UE8M0 scale bytes [R, K/32]."""
    v = np.abs(bf16_to_f64(w_bits))
    r, k = v.shape
    amax = v.reshape(r, k // MX_BLOCK, MX_BLOCK).max(axis=2)
    e = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    # floor(log2(amax)) exactly: frexp gives amax = f * 2^x with f in [0.5, 1), so floor(log2) = x - 1.
    _, x = np.frexp(amax[nz])
    e[nz] = np.clip(x.astype(np.int64) - 1 - E2M1_EMAX + 127, 0, 254)
    return e.astype(np.uint8)


def element_codes(w_bits: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """R17: E2M1 codes [R, K] (sign | nearest magnitude of |v| / 2^(E - 127), ties even, saturating)."""
    v = bf16_to_f64(w_bits)
    r, k = v.shape
    scale = np.repeat(UE8M0_TABLE[scale_bytes.astype(np.int64)], MX_BLOCK, axis=1)
    q = np.abs(v) / scale                               # exact: a power-of-two scaling in float64
    # magnitude code: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (lhs vs midpoints, rhs factor 1)
    mag = _nearest_code_ties_even(q, _E2M1_MIDS, np.ones_like(q))
    sign = (np.asarray(w_bits, dtype=np.uint16) >> 15).astype(np.uint8)
    return (sign << 3) | mag.astype(np.uint8)


def quantize(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """R17/R18: BF16 [R, K] (K a multiple of 32) -> (packed uint8 [R, K/2], scales uint8 [R, K/32])."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 2 or w_bits.shape[1] % MX_BLOCK:
        raise ValueError("MXFP4 needs [R, K] with K a multiple of 32")
    sb = block_scale_bytes(w_bits)
    return pack_nibbles(element_codes(w_bits, sb)), sb


def dequant_exact(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 values as float64 [R, K]: E2M1 * 2^(E - 127), exact."""
    codes = unpack_nibbles(packed)
    return E2M1_TABLE[codes] * np.repeat(UE8M0_TABLE[np.asarray(scales, dtype=np.int64)], MX_BLOCK, axis=1)


def linear_w4a4_ref(x_bits: np.ndarray, w_packed: np.ndarray, w_scales: np.ndarray):
    """R19: (y_ref, bound) float64 [M, N]: X quantized to MXFP4 (R17), times the MXFP4 weight."""
    xp, xs = quantize(x_bits)
    xq = dequant_exact(xp, xs)
    wq = dequant_exact(w_packed, w_scales)
    return xq @ wq.T, np.abs(xq) @ np.abs(wq).T


def linear_w4a4_violations(y: np.ndarray, y_ref: np.ndarray, bound: np.ndarray) -> np.ndarray:
    """R19's acceptance: the same form as the W4A16 linear's (FP32 accumulation, BF16 output)."""
    return linear_violations(y, y_ref, bound)
