"""Seeded synthetic inputs for the NVFP4 weight-only linear.

This module holds the workload shapes and the random-input recipes only.  It
contains none of the NVFP4 arithmetic: no scale choice, no rounding to E2M1 or
E4M3, no dequantization.  Both the CPU oracle side (in the tests) and the GPU
side consume the same BF16 bit patterns produced here, so an input never comes
from either implementation.

BF16 tensors are returned as ``numpy.uint16`` arrays of raw bit patterns,
produced by rounding float32 normals to bfloat16 (round to nearest even, as
torch's CPU cast does).

Shapes and statistics follow the model card of the 27B W4A16 NVFP4 checkpoint
(page "Qwen3.8-27B-NVFP4 (compressed-tensors)": linear weights NVFP4 with group
size 16, activations left in BF16, merged gate/up members sharing one tensor
scale with an amax spread of 3.7x) and the engine's decode/prefill workloads
(tg128 -> M=1, pp512 -> M=512, pp4096-class long prefill -> M=2048).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

# Seeds of every synthetic input.
SEED_W = 0          # weights
SEED_X = 1          # activations
SEED_OUTLIER = 2    # which input columns are outliers (decode workload)
SEED_UP = 3         # the "up" half of the merged gate/up weight
SEED_ROUTE = 4      # expert choices of the routed workloads
SEED_KV = 5         # KV-cache lengths (5), page order (6) and contents (7)

W_STD = 0.02
X_STD = 1.0
OUTLIER_FRACTION = 0.01
OUTLIER_GAIN = 8.0          # power of two: exact in BF16
GATE_UP_AMAX_RATIO = 3.7    # amax(gate) / amax(up), the spread the model card reports


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round a float32 array to bfloat16 (RNE, torch's CPU cast); return the uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape: Tuple[int, ...], std: float, seed: int) -> np.ndarray:
    """Seeded N(0, std^2) samples (PCG64, float32) rounded to BF16 bits."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_bits_from_f32(a)


def outlier_columns(k: int, seed: int = SEED_OUTLIER, fraction: float = OUTLIER_FRACTION) -> np.ndarray:
    """round(fraction*k) distinct input columns, drawn without replacement, sorted."""
    n = int(round(fraction * k))
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(k, size=n, replace=False))


def weight_plain(n: int, k: int, seed: int = SEED_W, std: float = W_STD) -> np.ndarray:
    return normal_bf16((n, k), std, seed)


def weight_with_outlier_columns(n: int, k: int, seed: int = SEED_W) -> np.ndarray:
    """~N(0, 0.02^2) weights whose outlier input columns are multiplied by 8 (before BF16 rounding)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, k), dtype=np.float32)
    a *= np.float32(W_STD)
    cols = outlier_columns(k)
    a[:, cols] *= np.float32(OUTLIER_GAIN)
    return bf16_bits_from_f32(a)


def weight_gate_up(n_half: int, k: int) -> Tuple[np.ndarray, np.ndarray, float]:
    """Gate and up halves of a merged gate/up weight.

    Gate ~N(0, 0.02^2) (seed 0).  Up is drawn independently (seed 3) and rescaled
    in float32, before BF16 rounding, so that amax(gate)/amax(up) is about 3.7.
    Returns (gate_bits, up_bits, exact post-rounding amax ratio).
    """
    gate = weight_plain(n_half, k, SEED_W)
    amax_gate = float(np.abs(f32_from_bf16_bits(gate)).max())
    rng = np.random.default_rng(SEED_UP)
    up = rng.standard_normal((n_half, k), dtype=np.float32)
    up *= np.float32(amax_gate / GATE_UP_AMAX_RATIO / float(np.abs(up).max()))
    up_bits = bf16_bits_from_f32(up)
    amax_up = float(np.abs(f32_from_bf16_bits(up_bits)).max())
    return gate, up_bits, amax_gate / amax_up


def activations(m: int, k: int, seed: int = SEED_X) -> np.ndarray:
    return normal_bf16((m, k), X_STD, seed)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic linear problem: Y[m, n] = X[m, :] . W_hat[n, :]."""
    name: str
    description: str
    n: int
    k: int
    ms: Tuple[int, ...]
    weight_kind: str            # "plain" | "outliers" | "gate_up"

    def weight(self) -> np.ndarray:
        """BF16 bits of the (merged) weight, shape [n, k]."""
        if self.weight_kind == "plain":
            return weight_plain(self.n, self.k)
        if self.weight_kind == "outliers":
            return weight_with_outlier_columns(self.n, self.k)
        if self.weight_kind == "gate_up":
            g, u, _ = weight_gate_up(self.n // 2, self.k)
            return np.concatenate([g, u], axis=0)
        raise ValueError(self.weight_kind)

    def activations(self, m: Optional[int] = None) -> np.ndarray:
        return activations(self.ms[0] if m is None else m, self.k)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", "tiny NVFP4 linear: W 256x512 ~N(0,0.02), X 1x512 ~N(0,1)",
                 256, 512, (1,), "plain"),
        Workload("decode", "decode GEMV: M=1, N=5120, K=5120, 1% outlier input columns x8",
                 5120, 5120, (1,), "outliers"),
        Workload("gate_up", "merged gate/up GEMV: M=1, N=2x17408, K=5120, amax ratio 3.7, one shared tensor scale",
                 2 * 17408, 5120, (1,), "gate_up"),
        Workload("small_m_up", "batched decode: M in {8,32}, N=17408, K=5120",
                 17408, 5120, (8, 32), "plain"),
        Workload("small_m_down", "batched decode down projection: M in {8,32}, N=5120, K=17408",
                 5120, 17408, (8, 32), "plain"),
        Workload("prefill", "prefill GEMM: M in {512,2048}, N=17408, K=5120",
                 17408, 5120, (512, 2048), "plain"),
        Workload("prefill_down", "prefill GEMM, down projection: M in {512,2048}, N=5120, K=17408",
                 5120, 17408, (512, 2048), "plain"),
    ]
}


def workload_names() -> List[str]:
    return list(WORKLOADS)


@dataclasses.dataclass(frozen=True)
class MoeWorkload:
    """Synthetic routed linear over an expert stack: t tokens, each routed to topk of `experts` matrices [n, k].

    The stack is built from one seeded ~N(0, 0.02) matrix, expert i scaled by (1 + i / 64) (so every expert
    has its own tensor scale); route r of a rotation of `experts / topk` routes sends the token to experts
    r * topk .. r * topk + topk - 1, so consecutive calls read different experts.
    """
    name: str
    description: str
    experts: int
    n: int
    k: int
    topk: int
    t: int = 1

    def base_weight(self) -> np.ndarray:
        return weight_plain(self.n, self.k)

    def routes(self) -> np.ndarray:
        """int32 [experts // topk, t, topk]."""
        r = np.arange(self.experts // self.topk, dtype=np.int32)[:, None, None] * self.topk
        return (r + np.arange(self.topk, dtype=np.int32)[None, None, :]).repeat(self.t, axis=1).astype(np.int32)

    def expert_scale(self, i: int) -> float:
        """Expert i's weight = BF16(base * (1 + i / 64)) (the factor is exact in FP32)."""
        return 1.0 + i / 64.0

    def expert_weight(self, i: int, base: np.ndarray = None) -> np.ndarray:
        """BF16 bits of expert i: the FP32 product base * expert_scale(i), rounded to nearest even."""
        base = self.base_weight() if base is None else base
        return bf16_bits_from_f32(f32_from_bf16_bits(base) * np.float32(self.expert_scale(i)))

    def random_routes(self, seed: int = SEED_ROUTE) -> np.ndarray:
        """int32 [t, topk]: each token's topk distinct experts, uniform at random (a balanced router)."""
        rng = np.random.default_rng(seed)
        return np.argsort(rng.random((self.t, self.experts)), axis=1)[:, :self.topk].astype(np.int32)


MOE_DECODE = MoeWorkload("moe_decode", "routed MoE decode: 128 experts of N=2048, K=4096, top-8, one token",
                         experts=128, n=2048, k=4096, topk=8)
MOE_PREFILL = MoeWorkload("moe_prefill", "grouped MoE prefill: 2048 tokens, each routed to 8 of 128 experts "
                          "of N=2048, K=4096", experts=128, n=2048, k=4096, topk=8, t=2048)


@dataclasses.dataclass(frozen=True)
class KvWorkload:
    """Synthetic paged FP4 KV cache and the gather of a chunked-prefill step.

    `seqs` sequences with seeded context lengths uniform in [min_len, max_len]; their pages are a random
    permutation of the cache's pages (a fragmented cache) plus `spare_pages` unused ones; output rows of
    sequence s start at dst_start[s], with `chunk` rows left free after each sequence for its current chunk.
    Codes are uniform random bytes (every E2M1 nibble); scale bytes are E4M3 codes drawn around 1/8 .. 8
    (0x28..0x48, NVFP4) or UE8M0 exponents 120..134 (MXFP4); the NVFP4 tensor scale is 1/64.
    """
    name: str
    description: str
    seqs: int
    heads: int
    head_dim: int
    block_size: int
    min_len: int
    max_len: int
    chunk: int
    spare_pages: int = 64

    def seq_lens(self) -> np.ndarray:
        rng = np.random.default_rng(SEED_KV)
        return rng.integers(self.min_len, self.max_len + 1, size=self.seqs).astype(np.int32)

    def layout(self):
        """(block_table int32 [seqs, max_blocks] (-1 past each sequence's pages), seq_lens, dst_start, num_blocks,
        out_rows)."""
        lens = self.seq_lens()
        pages = (lens + self.block_size - 1) // self.block_size
        max_blocks = int(pages.max())
        num_blocks = int(pages.sum()) + self.spare_pages
        perm = np.random.default_rng(SEED_KV + 1).permutation(num_blocks).astype(np.int32)
        table = np.full((self.seqs, max_blocks), -1, dtype=np.int32)
        at = 0
        for s in range(self.seqs):
            table[s, :pages[s]] = perm[at:at + pages[s]]
            at += int(pages[s])
        dst = np.concatenate([[0], np.cumsum(lens.astype(np.int64) + self.chunk)[:-1]]).astype(np.int32)
        out_rows = int(dst[-1]) + int(lens[-1]) + self.chunk
        return table, lens, dst, num_blocks, out_rows

    def cache(self, fmt: str, num_blocks: int):
        """(codes uint8 [num_blocks, block_size, heads, head_dim/2], scales uint8 [..., head_dim/G])."""
        g = 16 if fmt == "nvfp4" else 32
        rng = np.random.default_rng(SEED_KV + 2)
        codes = rng.integers(0, 256, size=(num_blocks, self.block_size, self.heads, self.head_dim // 2),
                             dtype=np.uint8)
        lo, hi = (0x28, 0x48) if fmt == "nvfp4" else (120, 134)
        scales = rng.integers(lo, hi + 1, size=(num_blocks, self.block_size, self.heads, self.head_dim // g),
                              dtype=np.uint8)
        return codes, scales

    KV_TSCALE = 1.0 / 64.0


KV_PREFILL = KvWorkload("kv_gather", "paged FP4 KV gather for chunked prefill: 16 sequences of 1024..8192 past "
                        "tokens, 8 KV heads x 128, 16-token pages", seqs=16, heads=8, head_dim=128, block_size=16,
                        min_len=1024, max_len=8192, chunk=512)
