"""CPU oracle for the NVFP4 weight-only (W4A16) linear.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python binding)
never calls it, and it shares no code, table or helper with the HIP path.

Everything here is plain numpy in float64 (with torch CPU used only for the
float32 -> bfloat16 round-to-nearest-even cast).  Each decision that turns a
real number into an integer code is taken exactly: both sides of every
comparison are short products that float64 represents without rounding.

Sources (web pages, cited by title and section):
  * "Raphael Friedmann" homepage, NVFP4 bit diagram: an E2M1 element is one
    sign bit, two exponent bits and one mantissa bit (sixteen values), with an
    FP8 scale per 16 values and an FP32 scale per tensor; the range comes from
    the two scales.
  * imp "docs/quantization.md", imp-quantize section: the checkpoint holds
    packed nibbles (U8), F8_E4M3 micro-scales and an F32 tensor scale; the
    scales are plain round-to-nearest over the weights, with no calibration.
  * same page, the paragraph on searching micro-scales: the micro-scale is
    taken from the block absmax; the E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3,
    4, 6.
  * model card "Qwen3.8-27B-NVFP4 (compressed-tensors)", "What is quantized":
    weight-only (activations stay BF16), group size 16; merged q/k/v and
    gate/up members share one tensor scale.

Readings taken where the pages are silent or open:
  R1 tensor scale   tscale = fl32(amax / 2688), 2688 = 6 * 448, stored as a multiplier.
  R2 micro-scale    the E4M3 value nearest to the real number 448*bam/amax.
  R3 element        the E2M1 magnitude nearest to the real 2688*|w|/(amax*s), saturating at 6.
  R4 ties           to the even code, for both E4M3 and E2M1.
  R5 sign           the BF16 sign bit (so -0.0 and tiny negatives give code 0x8).
  R6 zero           bam = 0 -> scale code 0; scale 0 -> magnitude 0; amax = 0 -> tscale = +0.
  R7 nibble order   element 2j in the low nibble, 2j+1 in the high nibble of byte j.
  R8 layouts        W, packed and scales are row-major [N, K], [N, K/2], [N, K/16]; blocks run along K.
  R9 dequant        w_hat = RNE_bf16(fl32(fl32(E2M1 * E4M3) * tscale)).
  R10 linear        Y[m, n] = sum_k X[m, k] * E2M1 * E4M3 * tscale, accepted within 2e-3 * sum_k |X * w_hat|.
  R11 output        the linear's output is BF16: on top of R10, the final rounding to BF16 may add up to
                    2^-8 of the output's magnitude.
  R12 expert stack  imp "docs/quantization.md", NVFP4 kernel pipeline, MoE layers: per-expert weights
                    become one contiguous [ne, N, K_packed] buffer per layer and projection.  Each expert
                    is its own quantized tensor with its own tensor scale (matrix i of the stack is
                    quantize(W[i])).
  R13 routed        y[t, j] = X[t] . W_hat[route[t, j]]^T for top-k routing (each token's k chosen experts);
                    an expert id outside [0, ne) gives a zero row.
  R20 NVFP4 x NVFP4 imp "docs/quantization.md", the Modelopt row of the loader table: a prefill in which
                    the activations are NVFP4 too.  The pages do not say how the activation scales are
                    chosen; the plain reading is this module's own quantizer applied to X [M, K] (one tensor
                    scale from max |X| over the whole call, an E4M3 scale per 16 along K, R1-R8), then
                    Y = X_hat . W_hat^T, accepted like R10/R11 with the bound sum_k |x_hat * w_hat|.

Parity pins: every function here is checked by tests/test_oracle_pins.py
against values the pages print, library routines (torch float8_e4m3fn),
exact-rational brute force and closed-form invariants.  No function is
"parity unpinned".
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
import torch

BLOCK = 16                 # elements per micro-scale (group size 16)
E2M1_MAX = 6.0             # largest E2M1 magnitude
E4M3_MAX = 448.0           # largest finite E4M3 value (OCP OFP8 E4M3FN)
SCALE_DENOM = E2M1_MAX * E4M3_MAX   # 2688


# --------------------------------------------------------------------------
# Tables built from the bit layouts.
# --------------------------------------------------------------------------
def _e2m1_from_bits(code: int) -> float:
    """E2M1 nibble s|e1 e0|m: exponent bias 1, e=0 is subnormal (m * 0.5)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    return -mag if s else mag


def _e4m3_from_bits(code: int) -> float:
    """OCP E4M3FN byte s|eeee|mmm: bias 7, e=0 subnormal m/8 * 2^-6, 0x7F/0xFF NaN, no infinities."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


E2M1_TABLE = np.array([_e2m1_from_bits(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([_e4m3_from_bits(c) for c in range(256)], dtype=np.float64)

# Non-negative finite E4M3 values in code order (codes 0x00..0x7E) and E2M1 magnitudes (codes 0..7).
_E4M3_POS = E4M3_TABLE[:0x7F]
_E2M1_POS = E2M1_TABLE[:8]


# --------------------------------------------------------------------------
# BF16 helpers (bit patterns as uint16).
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bits, round to nearest even (torch's CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _nearest_code_ties_even(lhs: np.ndarray, mids: np.ndarray, rhs_factor: np.ndarray) -> np.ndarray:
    """Index of the nearest grid point, ties to the even index.

    The grid is implicit: ``mids[c]`` is the midpoint between grid points c and
    c+1, and the real number being rounded is ``lhs / rhs_factor``.  The point
    lies above midpoint c when lhs > mids[c] * rhs_factor (c even: a tie stays
    on the even point c) or lhs >= mids[c] * rhs_factor (c odd: a tie moves up
    to the even point c+1).  The index is the number of midpoints it lies
    above.  All products are exact in float64 for the operands used here.
    """
    code = np.zeros(np.shape(lhs), dtype=np.int64)
    for c, u in enumerate(mids):
        rhs = u * rhs_factor
        code += (lhs > rhs) if (c % 2 == 0) else (lhs >= rhs)
    return code


_E4M3_MIDS = (_E4M3_POS[:-1] + _E4M3_POS[1:]) / 2.0   # 126 midpoints, exact in float64
_E2M1_MIDS = (_E2M1_POS[:-1] + _E2M1_POS[1:]) / 2.0   # 0.25 0.75 1.25 1.75 2.5 3.5 5


# --------------------------------------------------------------------------
# Quantizer (imp-quantize: round-to-nearest, absmax micro-scale).
# --------------------------------------------------------------------------
def tensor_amax(w_bits: np.ndarray) -> float:
    """amax = max |w| over the whole tensor (exact)."""
    w = bf16_to_f64(w_bits)
    return float(np.abs(w).max()) if w.size else 0.0


def tensor_scale(amax: float) -> np.float32:
    """R1: tscale = fl32(amax / 2688), IEEE binary32 division."""
    return np.float32(amax) / np.float32(SCALE_DENOM)


def block_scale_codes(w_bits: np.ndarray, amax: float) -> np.ndarray:
    """R2/R4/R6: per row and per 16 consecutive K elements, the E4M3 code nearest to 448*bam/amax."""
    w = np.abs(bf16_to_f64(w_bits))
    n, k = w.shape
    bam = w.reshape(n, k // BLOCK, BLOCK).max(axis=2)
    if amax == 0.0:
        return np.zeros((n, k // BLOCK), dtype=np.uint8)
    # Compare 448*bam against u*amax: both exact in float64.
    code = _nearest_code_ties_even(E4M3_MAX * bam, _E4M3_MIDS, np.float64(amax))
    return code.astype(np.uint8)


def element_codes(w_bits: np.ndarray, scale_codes: np.ndarray, amax: float) -> np.ndarray:
    """R3/R4/R5: the 4-bit code of each element, sign from the BF16 sign bit."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    n, k = w_bits.shape
    w = np.abs(bf16_to_f64(w_bits))
    s = np.repeat(E4M3_TABLE[scale_codes.astype(np.int64)], BLOCK, axis=1)  # per-element block scale
    # Compare 2688*|w| against t*(amax*s): both exact in float64.
    mag = _nearest_code_ties_even(SCALE_DENOM * w, _E2M1_MIDS, np.float64(amax) * s)
    mag[s == 0.0] = 0
    sign = (w_bits >> 15).astype(np.int64)
    return ((sign << 3) | mag).astype(np.uint8)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """R7: byte j of a row = code[2j] | code[2j+1] << 4."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    n, kh = packed.shape
    codes = np.empty((n, 2 * kh), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    return codes


def quantize(w_bits: np.ndarray, amax: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray, np.float32]:
    """BF16 [N, K] -> (packed uint8 [N, K/2], scales uint8 [N, K/16], tscale float32).

    ``amax`` overrides the tensor's own absmax; it is how members of a merged
    linear (q/k/v, gate/up) are quantized against one shared tensor scale.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 2 or w_bits.shape[1] % BLOCK != 0:
        raise ValueError("W must be [N, K] with K a multiple of 16")
    if not np.all(np.isfinite(bf16_to_f64(w_bits))):
        raise ValueError("W must be finite")
    if amax is None:
        amax = tensor_amax(w_bits)
    scales = block_scale_codes(w_bits, amax)
    codes = element_codes(w_bits, scales, amax)
    return pack_nibbles(codes), scales, tensor_scale(amax)


def quantize_shared(members) -> Tuple[list, np.float32]:
    """Quantize the members of a merged linear against one tensor scale (the max of their amaxes)."""
    amax = max(tensor_amax(m) for m in members)
    outs = [quantize(m, amax=amax) for m in members]
    return [(p, s) for p, s, _ in outs], tensor_scale(amax)


# --------------------------------------------------------------------------
# Dequantization and the linear.
# --------------------------------------------------------------------------
def decoded_products(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E2M1(code) * E4M3(scale) per element, float64 (exact: at most 6 significant bits)."""
    codes = unpack_nibbles(packed)
    s = np.repeat(E4M3_TABLE[np.asarray(scales, dtype=np.int64)], BLOCK, axis=1)
    return E2M1_TABLE[codes.astype(np.int64)] * s


def dequant(packed: np.ndarray, scales: np.ndarray, tscale) -> np.ndarray:
    """R9: BF16 bits of RNE_bf16(fl32(fl32(E2M1 * E4M3) * tscale))."""
    prod32 = decoded_products(packed, scales).astype(np.float32)   # exact
    w32 = prod32 * np.float32(tscale)                              # one binary32 rounding
    return f32_to_bf16_rne(w32)


def dequant_exact(packed: np.ndarray, scales: np.ndarray, tscale) -> np.ndarray:
    """E2M1 * E4M3 * tscale in float64 (exact: at most 2 + 4 + 24 significant bits)."""
    return decoded_products(packed, scales) * np.float64(np.float32(tscale))


def linear_ref(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, tscale) -> Tuple[np.ndarray, np.ndarray]:
    """R10: (y_ref, bound) with y_ref = X . W_hat^T and bound = |X| . |W_hat|^T, both float64 [M, N]."""
    x = bf16_to_f64(x_bits)
    w = dequant_exact(packed, scales, tscale)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def linear_w4a4_ref(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray, tscale,
                    x_amax: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """R20: (y_ref, bound) float64 [M, N]; X is quantized to NVFP4 (its own tensor scale) before the product.

    x_amax: max |X| of the whole activation tensor when x_bits holds only some of its rows."""
    xp, xs, xts = quantize(np.asarray(x_bits, dtype=np.uint16), amax=x_amax)
    x = dequant_exact(xp, xs, xts)
    w = dequant_exact(packed, scales, tscale)
    return x @ w.T, np.abs(x) @ np.abs(w).T


LINEAR_TOL = 2e-3
BF16_UNIT_ROUNDOFF = 2.0 ** -8   # 8 significant bits: RNE to BF16 moves a value by at most 2^-8 of it


def linear_violations(y: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, tol: float = LINEAR_TOL,
                      out_roundoff: float = BF16_UNIT_ROUNDOFF) -> np.ndarray:
    """Boolean mask of outputs outside the accepted error.

    R11: the accumulation must stay within tol * bound of the exact sum
    (bound = sum_k |x * w_hat|), and the output may then be rounded to BF16,
    which the W4A16 output format imposes and which alone can move it by up to
    2^-8 of its magnitude (more than tol * bound when one term dominates).  So:
        |y - y_ref| <= tol * bound + 2^-8 * (|y_ref| + tol * bound).
    bound = 0 requires y = 0.
    """
    y = np.asarray(y, dtype=np.float64)
    acc = tol * bound
    return ~(np.abs(y - y_ref) <= acc + out_roundoff * (np.abs(y_ref) + acc))


# --------------------------------------------------------------------------
# Expert stacks (mixture-of-experts layers).
# --------------------------------------------------------------------------
def quantize_experts(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """R12: BF16 [E, N, K] -> (packed [E, N, K/2], scales [E, N, K/16], tscale float32 [E]), one tensor per expert."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 3:
        raise ValueError("W must be [E, N, K]")
    outs = [quantize(w_bits[i]) for i in range(w_bits.shape[0])]
    return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]),
            np.array([o[2] for o in outs], dtype=np.float32))


def dequant_experts(packed: np.ndarray, scales: np.ndarray, tscale: np.ndarray) -> np.ndarray:
    """R9 applied to every matrix of a stack: BF16 bits [E, N, K]."""
    return np.stack([dequant(packed[i], scales[i], tscale[i]) for i in range(packed.shape[0])])


def linear_routed_ref(x_bits: np.ndarray, route: np.ndarray, packed: np.ndarray, scales: np.ndarray,
                      tscale: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """R13: (y_ref, bound), float64 [T, topk, N]; pairs routed to an expert outside [0, E) are zero."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    route = np.asarray(route, dtype=np.int64)
    t_count, topk = route.shape
    e_count, n = packed.shape[0], packed.shape[1]
    y = np.zeros((t_count, topk, n))
    bound = np.zeros((t_count, topk, n))
    for e in range(e_count):
        ts, js = np.nonzero(route == e)
        if ts.size == 0:
            continue
        ye, be = linear_ref(x_bits[ts], packed[e], scales[e], tscale[e])
        y[ts, js] = ye
        bound[ts, js] = be
    return y, bound
