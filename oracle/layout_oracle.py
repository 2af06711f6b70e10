"""CPU oracle of the library's kernel-native weight layout.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product path never calls it, and it shares no code with
the HIP path.

The pages describe a loader that keeps the checkpoint's packed NVFP4 weights
for decode and re-lays scale factors once for the prefill GEMM (imp
"docs/quantization.md", "NVFP4 kernel pipeline", Dense layers: registered in
the decode cache without re-quantization, then a scale-factor re-layout for
prefill).  The layout below is this library's own re-layout of the same bytes
(values unchanged), in the order its MI355X kernels read them.  The pages do not
define it; it is specified here and in include/nvfp4.h, and pinned by a
hand-written fixture (tests/golden/kernel_native_layout.txt).

Definition, for a weight [N, K] with K a multiple of 128 (packed [N, K/2],
scales [N, K/16], element 2j of a row in the low nibble of packed byte j):
  * rows are grouped in tiles of 16 (N padded with zero rows to a multiple of
    16; tiles = ceil(N / 16)), K in quads of 128 elements;
  * block (tile t, quad q) is 1152 bytes at offset (q * tiles + t) * 1152
    (quad-major: all tiles of quad 0, then all tiles of quad 1, ...);
  * its first 1024 bytes are 64 slots of 16 bytes; slot s = 16 g + r
    (g = 0..3, r = 0..15) holds, as four 4-byte words i = 0..3, the elements
        k = 128 q + 32 i + 8 g + e,  e = 0..7,
    of row 16 t + r, in the canonical nibble order (element e of word i in
    nibble e, low nibble first);
  * its last 128 bytes are 32 words; word 16 h + r (h = 0, 1) holds, as byte
    i = 0..3, the E4M3 scale of block 8 q + 2 i + h of row 16 t + r (the block
    covering elements 128 q + 32 i + 16 h .. + 16).
So the 8 elements of slot s, word i (k = 128 q + 32 i + 8 g + e) have the
scale in byte i of word 16 (g // 2) + r.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

TILE_ROWS = 16
QUAD_K = 128
BLOCK_BYTES = 1152          # 1024 packed + 128 scale bytes per (tile, quad)


def prepared_bytes(n: int, k: int) -> int:
    if n <= 0 or k <= 0 or k % QUAD_K != 0:
        raise ValueError("kernel-native layout needs n > 0 and k a positive multiple of 128")
    tiles = -(-n // TILE_ROWS)
    return tiles * (k // QUAD_K) * BLOCK_BYTES


def _codes(packed: np.ndarray) -> np.ndarray:
    """Canonical packed [N, K/2] -> 4-bit codes [N, K] (element 2j low nibble of byte j)."""
    p = np.asarray(packed, dtype=np.uint8)
    c = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.uint8)
    c[:, 0::2] = p & 0xF
    c[:, 1::2] = p >> 4
    return c


def prepare(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Canonical (packed [N, K/2], scales [N, K/16]) -> the kernel-native byte array, element by element."""
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, k = packed.shape[0], 2 * packed.shape[1]
    out = np.zeros(prepared_bytes(n, k), dtype=np.uint8)
    codes = _codes(packed)
    quads, tiles = k // QUAD_K, -(-n // TILE_ROWS)
    for row in range(n):
        t, r = divmod(row, TILE_ROWS)
        for q in range(quads):
            base = (q * tiles + t) * BLOCK_BYTES
            for g in range(4):
                for i in range(4):
                    k0 = QUAD_K * q + 32 * i + 8 * g
                    word = 0
                    for e in range(8):
                        word |= int(codes[row, k0 + e]) << (4 * e)
                    off = base + 16 * (16 * g + r) + 4 * i
                    out[off:off + 4] = np.frombuffer(np.uint32(word).tobytes(), dtype=np.uint8)
            for h in range(2):
                for i in range(4):
                    out[base + 1024 + 4 * (16 * h + r) + i] = scales[row, 8 * q + 2 * i + h]
    return out


def unprepare(prep: np.ndarray, n: int, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """The kernel-native byte array -> canonical (packed [N, K/2], scales [N, K/16]); padding rows dropped."""
    prep = np.asarray(prep, dtype=np.uint8)
    if prep.size != prepared_bytes(n, k):
        raise ValueError("size does not match n, k")
    quads, tiles = k // QUAD_K, -(-n // TILE_ROWS)
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // 16), dtype=np.uint8)
    for row in range(n):
        t, r = divmod(row, TILE_ROWS)
        for q in range(quads):
            base = (q * tiles + t) * BLOCK_BYTES
            for g in range(4):
                for i in range(4):
                    off = base + 16 * (16 * g + r) + 4 * i
                    word = int(np.frombuffer(prep[off:off + 4].tobytes(), dtype=np.uint32)[0])
                    k0 = QUAD_K * q + 32 * i + 8 * g
                    for e in range(8):
                        codes[row, k0 + e] = (word >> (4 * e)) & 0xF
            for h in range(2):
                for i in range(4):
                    scales[row, 8 * q + 2 * i + h] = prep[base + 1024 + 4 * (16 * h + r) + i]
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def padding_is_zero(prep: np.ndarray, n: int, k: int) -> bool:
    """Rows n .. 16 * ceil(n / 16) - 1 of the last tile hold zero codes and zero scales."""
    prep = np.asarray(prep, dtype=np.uint8)
    quads, tiles = k // QUAD_K, -(-n // TILE_ROWS)
    t = (n - 1) // TILE_ROWS
    for row in range(n, (t + 1) * TILE_ROWS):
        r = row - t * TILE_ROWS
        for q in range(quads):
            base = (q * tiles + t) * BLOCK_BYTES
            for g in range(4):
                off = base + 16 * (16 * g + r)
                if prep[off:off + 16].any():
                    return False
            for h in range(2):
                off = base + 1024 + 4 * (16 * h + r)
                if prep[off:off + 4].any():
                    return False
    return True
