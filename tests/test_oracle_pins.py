"""Pins for the CPU oracle: checked against the pages, a library, exact rationals and invariants.

None of these tests re-types the oracle's own formula.  Each pin reaches the
expected value by another route:
  * the E2M1 magnitudes printed on the pages (tests/golden/e2m1_magnitudes.txt);
  * torch's float8_e4m3fn (an independent OCP E4M3FN implementation) for the
    E4M3 table and for round-to-nearest-even onto the E4M3 grid;
  * exhaustive nearest-point search in exact rational arithmetic (fractions)
    on tiny inputs;
  * closed-form facts (block absmax maps to +-6, idempotence, the shared-scale
    identity of merged linears, amax recovery from the tensor scale).
The mutation tests at the end plant plausible mistakes in the oracle and
check that some pin fails.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from nvfp4_weight_only_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(line)
    return vals


def _bits(values):
    return WL.bf16_bits_from_f32(np.asarray(values, dtype=np.float32))


# --------------------------------------------------------------------------
# Pin functions (also reused by the mutation tests).
# --------------------------------------------------------------------------
def pin_e2m1_table():
    mags = [float(v) for v in _read_golden("e2m1_magnitudes.txt")]
    assert len(mags) == 8
    assert list(O.E2M1_TABLE[:8]) == mags
    assert list(-O.E2M1_TABLE[8:]) == mags
    assert np.signbit(O.E2M1_TABLE[8]) and not np.signbit(O.E2M1_TABLE[0])


def pin_e4m3_table():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(O.E4M3_TABLE), nan_ref)
    assert np.array_equal(O.E4M3_TABLE[~nan_ref], ref[~nan_ref])
    assert np.array_equal(np.signbit(O.E4M3_TABLE[~nan_ref]), np.signbit(ref[~nan_ref]))


def pin_nibble_layout():
    # codes (1, 2) -> one byte 0x21 -> decoded [0.5, 1.0] (element 2j in the low nibble)
    codes = np.array([[1, 2, 0xF, 0x8]], dtype=np.uint8)
    packed = O.pack_nibbles(codes)
    assert packed.tolist() == [[0x21, 0x8F]]
    scales = np.array([[0x38]], dtype=np.uint8)   # E4M3 0x38 = 1.0
    w = O.decoded_products(np.pad(packed, ((0, 0), (0, 6))), scales)
    assert w[0, :4].tolist() == [0.5, 1.0, -6.0, -0.0]
    assert np.signbit(w[0, 3])


def _scales_via_torch(w_bits, amax):
    """E4M3 code of fl32(448*bam/amax) by torch's float32 -> float8_e4m3fn cast (RNE)."""
    w = np.abs(WL.f32_from_bf16_bits(w_bits).astype(np.float64))
    n, k = w.shape
    bam = w.reshape(n, k // 16, 16).max(axis=2)
    ratio = (np.float32(448.0) * bam.astype(np.float32)) / np.float32(amax)  # 448*bam exact in fp32
    return torch.from_numpy(ratio.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_scales_match_torch_rounding(w_bits):
    amax = O.tensor_amax(w_bits)
    got = O.block_scale_codes(w_bits, amax)
    ref = _scales_via_torch(w_bits, amax)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} scale codes differ"


def _nearest_even(x, grid):
    """Exhaustive nearest point of ``grid`` to Fraction x, ties to the even index."""
    best = None
    for i, g in enumerate(grid):
        d = abs(x - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


E4M3_GRID = [Fraction(v) for v in torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()]


def pin_quantize_brute_force(w_bits, amax_override=None):
    """Scale and element codes equal an exhaustive exact-rational nearest-point search."""
    mags = [Fraction(v) for v in _read_golden("e2m1_magnitudes.txt")]
    packed, scales, tscale = O.quantize(w_bits, amax=amax_override)
    codes = O.unpack_nibbles(packed)
    w = [[Fraction(float(v)) for v in row] for row in WL.f32_from_bf16_bits(w_bits)]
    amax = Fraction(O.tensor_amax(w_bits)) if amax_override is None else Fraction(amax_override)
    assert float(tscale) == float(np.float32(float(amax) / 2688.0)) or amax == 0
    n, k = len(w), len(w[0])
    for r in range(n):
        for b in range(k // 16):
            blk = w[r][16 * b:16 * b + 16]
            bam = max(abs(v) for v in blk)
            exp_s = 0 if amax == 0 else _nearest_even(448 * bam / amax, E4M3_GRID)
            assert scales[r, b] == exp_s, (r, b, scales[r, b], exp_s)
            s = E4M3_GRID[exp_s]
            for j, v in enumerate(blk):
                mag = 0 if s == 0 else _nearest_even(2688 * abs(v) / (amax * s), mags)
                sign = 1 if np.signbit(float(v)) or (v == 0 and _neg_zero(w_bits[r, 16 * b + j])) else 0
                assert codes[r, 16 * b + j] == (sign << 3 | mag), (r, 16 * b + j, codes[r, 16 * b + j], sign, mag)


def _neg_zero(bits):
    return int(bits) == 0x8000


def pin_dequant_closed_form(packed, scales, tscale):
    """w_hat = bf16(f32(E2M1 * E4M3) * tscale), built from the page magnitudes and torch's E4M3."""
    mags = np.array([float(v) for v in _read_golden("e2m1_magnitudes.txt")], dtype=np.float32)
    e2m1 = np.concatenate([mags, -mags])
    e4m3 = torch.from_numpy(np.asarray(scales, dtype=np.uint8).copy()).view(torch.float8_e4m3fn).to(torch.float32)
    codes = torch.from_numpy(O.unpack_nibbles(packed).astype(np.int64))
    vals = torch.from_numpy(e2m1)[codes] * e4m3.repeat_interleave(16, dim=1)
    ref = (vals * torch.tensor(float(tscale), dtype=torch.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.dequant(packed, scales, tscale)
    assert np.array_equal(got, ref)


def pin_linear_brute_force(x_bits, packed, scales, tscale):
    mags = [Fraction(v) for v in _read_golden("e2m1_magnitudes.txt")]
    e2m1 = mags + [-m for m in mags]
    e4m3 = torch.from_numpy(np.asarray(scales, dtype=np.uint8).copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    codes = O.unpack_nibbles(packed)
    x = WL.f32_from_bf16_bits(x_bits).astype(np.float64)
    t = Fraction(float(np.float32(tscale)))
    y_ref, bound = O.linear_ref(x_bits, packed, scales, tscale)
    m, k = x.shape
    n = codes.shape[0]
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(x[i, kk]) * e2m1[codes[j, kk]] * Fraction(e4m3[j, kk // 16]) * t for kk in range(k))
            babs = sum(abs(Fraction(x[i, kk]) * e2m1[codes[j, kk]] * Fraction(e4m3[j, kk // 16]) * t) for kk in range(k))
            assert abs(Fraction(y_ref[i, j]) - exact) <= Fraction(1, 10 ** 12) * (babs + Fraction(1, 10 ** 30)), (i, j)
            assert abs(Fraction(bound[i, j]) - babs) <= Fraction(1, 10 ** 12) * (babs + Fraction(1, 10 ** 30)), (i, j)


# --------------------------------------------------------------------------
# Tiny inputs with crafted ties.
# --------------------------------------------------------------------------
def tiny_inputs():
    """Random tiny matrices plus rows that put elements and scales exactly on rounding midpoints."""
    cases = []
    for (n, k, seed) in [(2, 16, 10), (3, 32, 11), (4, 64, 12), (1, 48, 13)]:
        cases.append(WL.normal_bf16((n, k), 0.02, seed))
    # Ties on E2M1 midpoints: amax = 6 in block 0 gives scale 448 there, so q = 448*|w|*... choose
    # a block with bam = 6 (scale 448 exactly -> tscale*scale = 1): q = |w| exactly.
    row = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -0.0]
    # Second block: bam = 3 -> 448*3/6 = 224 (an E4M3 value) -> q = 2*|w|.
    row2 = [3.0, 0.125, 0.375, 0.625, 0.875, 1.25, 1.75, 2.5, 0.0, -0.0, 1e-30, -1e-30, 2.0, 0.1, 0.2, 0.3]
    cases.append(_bits([row + row2]))
    # Ties on E4M3 midpoints: amax = 448 and bam = midpoint u gives 448*bam/amax = u exactly.
    mids = (np.array(E4M3_GRID[:-1], dtype=np.float64) + np.array(E4M3_GRID[1:], dtype=np.float64)) / 2
    blocks = []
    for u in mids[::5]:
        blk = [0.0] * 16
        blk[3] = u
        blk[7] = -u / 3
        blocks.append(blk)
    blocks.append([448.0] + [0.0] * 15)
    cases.append(_bits([sum(blocks, [])]))
    return cases


def _ties_present(w_bits):
    """Count exact E2M1 midpoint ties (sanity: the tie cases really are ties)."""
    packed, scales, _ = O.quantize(w_bits)
    amax = O.tensor_amax(w_bits)
    s = np.repeat(O.E4M3_TABLE[scales.astype(np.int64)], 16, axis=1)
    w = np.abs(WL.f32_from_bf16_bits(w_bits).astype(np.float64))
    with np.errstate(divide="ignore", invalid="ignore"):
        q = 2688 * w / (amax * s)
    return int(np.isin(q, [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]).sum())


# --------------------------------------------------------------------------
# Tests.
# --------------------------------------------------------------------------
def test_e2m1_table_matches_page_magnitudes():
    pin_e2m1_table()


def test_e4m3_table_matches_torch_float8_e4m3fn():
    pin_e4m3_table()
    assert O.E4M3_TABLE[0x7E] == 448.0 and O.E4M3_TABLE[0x01] == 2.0 ** -9


def test_nibble_layout_example():
    pin_nibble_layout()


def test_layout_sizes_follow_pages():
    g = dict(line.split() for line in _read_golden("nvfp4_layout.txt"))
    g = {k: int(v) for k, v in g.items()}
    for wl in WL.WORKLOADS.values():
        n, k = wl.n, wl.k
        packed_bytes = n * k * g["element_bits"] // 8
        scale_bytes = n * k // g["block_elements"] * g["block_scale_bits"] // 8
        assert packed_bytes == n * k // g["elements_per_byte"]
        bits_per_weight = (8 * (packed_bytes + scale_bytes) + g["tensor_scale_bits"]) / (n * k)
        assert abs(bits_per_weight - (4 + 8 / 16 + 32 / (n * k))) < 1e-12
    w = WL.normal_bf16((5, 48), 0.02, 7)
    packed, scales, tscale = O.quantize(w)
    assert packed.shape == (5, 24) and packed.dtype == np.uint8
    assert scales.shape == (5, 3) and scales.dtype == np.uint8
    assert isinstance(tscale, np.float32)


@pytest.mark.parametrize("idx", range(6))
def test_quantize_brute_force_tiny(idx):
    w = tiny_inputs()[idx]
    pin_quantize_brute_force(w)


def test_tie_cases_really_tie():
    cases = tiny_inputs()
    assert _ties_present(cases[4]) >= 14


def test_scales_match_torch_e4m3_rounding_random():
    for wl_bits in [WL.normal_bf16((64, 512), 0.02, 0), WL.weight_with_outlier_columns(64, 5120)]:
        pin_scales_match_torch_rounding(wl_bits)


def test_scales_match_torch_e4m3_rounding_at_every_midpoint():
    mids = (np.array(E4M3_GRID[:-1], dtype=np.float64) + np.array(E4M3_GRID[1:], dtype=np.float64)) / 2
    rows = []
    for u in mids:
        blk = [0.0] * 16
        blk[5] = u
        rows.append(blk + [448.0] + [0.0] * 15)
    w = _bits(rows)
    pin_scales_match_torch_rounding(w)
    codes = O.block_scale_codes(w, 448.0)[:, 0]
    assert np.all(codes % 2 == 0)   # every exact midpoint went to the even neighbour


def test_amax_recovered_from_tensor_scale_for_every_bf16():
    """RNE_bf16(fl32(2688 * fl32(a / 2688))) == a for all 32639 positive finite BF16 a."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    a = WL.f32_from_bf16_bits(bits)
    t = a / np.float32(2688.0)
    back = (t * np.float32(2688.0)).astype(np.float32)
    back_bits = WL.bf16_bits_from_f32(back)
    assert np.array_equal(back_bits, bits)
    for ai in a[::997]:
        assert O.tensor_scale(float(ai)) == np.float32(ai) / np.float32(2688.0)


@pytest.mark.parametrize("kind", ["plain", "outliers"])
def test_block_absmax_maps_to_six(kind):
    w = WL.weight_plain(64, 5120) if kind == "plain" else WL.weight_with_outlier_columns(64, 5120)
    packed, scales, _ = O.quantize(w)
    codes = O.unpack_nibbles(packed).reshape(64, -1, 16)
    a = np.abs(WL.f32_from_bf16_bits(w)).reshape(64, -1, 16)
    argmax = a.argmax(axis=2)
    top = np.take_along_axis(codes, argmax[..., None], axis=2)[..., 0] & 7
    normal = scales >= 0x08
    assert normal.sum() > 0
    assert np.all(top[normal] == 7)


@pytest.mark.parametrize("kind", ["plain", "outliers"])
def test_quantize_dequant_idempotent(kind):
    w = WL.weight_plain(32, 5120) if kind == "plain" else WL.weight_with_outlier_columns(32, 5120)
    p1, s1, t1 = O.quantize(w)
    w2 = O.dequant(p1, s1, t1)
    p2, s2, t2 = O.quantize(w2)
    assert t2 == t1
    normal = s1 >= 0x08
    assert np.array_equal(s2[normal], s1[normal])
    c1 = O.unpack_nibbles(p1).reshape(32, -1, 16)[normal]
    c2 = O.unpack_nibbles(p2).reshape(32, -1, 16)[normal]
    assert np.array_equal(c1, c2)


def test_shared_scale_identity_and_wrong_scale_failure():
    gate, up, ratio = WL.weight_gate_up(48, 512)
    assert 3.5 < ratio < 3.9
    merged = np.concatenate([gate, up], axis=0)
    pm, sm, tm = O.quantize(merged)
    (pg, sg), (pu, su) = O.quantize_shared([gate, up])[0]
    _, ts = O.quantize_shared([gate, up])
    assert ts == tm
    assert np.array_equal(np.concatenate([pg, pu]), pm)
    assert np.array_equal(np.concatenate([sg, su]), sm)
    # The failure mode the model card warns about: U's codes decoded against U's own scale.
    x = WL.activations(2, 512)
    y_ref, bound = O.linear_ref(x, pu, su, tm)
    wrong_t = O.tensor_scale(O.tensor_amax(up))
    y_wrong, _ = O.linear_ref(x, pu, su, wrong_t)
    assert O.linear_violations(y_wrong, y_ref, bound).mean() > 0.9
    # U's own scale is smaller than the shared one by the amax spread.
    ratio_seen = np.median(np.abs(y_ref) / np.maximum(np.abs(y_wrong), 1e-30))
    assert abs(ratio_seen - ratio) / ratio < 0.02


def test_dequant_closed_form_random_and_edges():
    for w in [WL.weight_plain(16, 512), WL.weight_with_outlier_columns(16, 512), tiny_inputs()[4], tiny_inputs()[5]]:
        pin_dequant_closed_form(*O.quantize(w))


@pytest.mark.parametrize("shape", [(1, 2, 16), (2, 3, 32), (3, 2, 48)])
def test_linear_brute_force_tiny(shape):
    m, n, k = shape
    w = WL.normal_bf16((n, k), 0.02, 20 + k)
    x = WL.normal_bf16((m, k), 1.0, 30 + k)
    pin_linear_brute_force(x, *O.quantize(w))


def test_linear_unit_scales_is_plain_matvec():
    """With every block scale 1.0 and tscale 1, the linear is a matvec over the E2M1 values."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(7, 64)).astype(np.uint8)
    packed = O.pack_nibbles(codes)
    scales = np.full((7, 4), 0x38, dtype=np.uint8)     # E4M3 0x38 == 1.0
    x = WL.normal_bf16((3, 64), 1.0, 6)
    mags = [float(v) for v in _read_golden("e2m1_magnitudes.txt")]
    vals = torch.tensor(mags + [-v for v in mags], dtype=torch.float64)[torch.from_numpy(codes.astype(np.int64))]
    xt = torch.from_numpy(WL.f32_from_bf16_bits(x).astype(np.float64))
    ref = torch.matmul(xt, vals.T).numpy()
    y, _ = O.linear_ref(x, packed, scales, np.float32(1.0))
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_zero_sign_and_range_edges():
    # all-zero tensor (with a -0): tscale 0, scales 0, codes keep the sign bit only
    w = _bits([[0.0] * 15 + [-0.0]])
    p, s, t = O.quantize(w)
    assert t == 0 and s.tolist() == [[0]] and O.unpack_nibbles(p)[0].tolist() == [0] * 15 + [8]
    assert np.array_equal(O.dequant(p, s, t), w)
    # single nonzero element: it becomes +-6 * 448 * tscale, everything else 0
    w = _bits([[0.0] * 7 + [-0.0371] + [0.0] * 24])
    p, s, t = O.quantize(w)
    c = O.unpack_nibbles(p)[0]
    assert c[7] == 0xF and s[0, 0] == 0x7E and s[0, 1] == 0
    # a block far below amax gets a subnormal or zero scale
    w = _bits([[100.0] + [0.0] * 15 + [1e-3] + [0.0] * 15 + [1e-7] + [0.0] * 15])
    p, s, t = O.quantize(w)
    assert s[0, 0] == 0x7E and 0 < s[0, 1] < 0x08 and s[0, 2] == 0
    assert O.unpack_nibbles(p)[0, 32] == 0


def test_invalid_inputs_rejected():
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 24), dtype=np.uint16))
    with pytest.raises(ValueError):
        O.quantize(_bits([[np.inf] + [0.0] * 15]))


def test_linear_tolerance_gate():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    bound = np.array([[10.0, 10.0, 0.0]])
    # accumulation allowance 2e-3 * 10 = 0.02, plus 2^-8 * (|y_ref| + 0.02) for the BF16 output rounding
    allow = 0.02 + 2.0 ** -8 * (1.0 + 0.02)
    assert not O.linear_violations(np.array([[1.0 + 0.999 * allow, -2.0, 0.0]]), y_ref, bound).any()
    assert O.linear_violations(np.array([[1.0 + 1.001 * allow, -2.0, 0.0]]), y_ref, bound).tolist() == [[True, False, False]]
    assert O.linear_violations(np.array([[1.0, -2.0, 1e-30]]), y_ref, bound).tolist() == [[False, False, True]]


def test_exact_sum_rounded_to_bf16_always_passes():
    """A perfect implementation (exact sum, then RNE to BF16) passes even when one term dominates."""
    rng = np.random.default_rng(11)
    y_ref = rng.standard_normal((4, 4096)) * np.exp(rng.uniform(-20, 20, (4, 4096)))
    bound = np.abs(y_ref) * rng.uniform(1.0, 1.001, y_ref.shape)      # |y| ~ bound: no cancellation
    y_bf16 = WL.f32_from_bf16_bits(WL.bf16_bits_from_f32(y_ref.astype(np.float32))).astype(np.float64)
    assert np.abs(y_bf16 - y_ref).max() > 0  # the rounding is visible
    assert not O.linear_violations(y_bf16, y_ref, bound).any()
    # ...while two BF16 ulps away fails when |y| ~ bound
    ulp = 2.0 ** (np.floor(np.log2(np.abs(y_ref))) - 7)
    assert O.linear_violations(y_ref + 2 * ulp * np.sign(y_ref), y_ref, bound).all()


# --------------------------------------------------------------------------
# Mutation tests: plant a mistake in the oracle, check that some pin fails.
# --------------------------------------------------------------------------
def _expect_pin_failure(monkeypatch, target, replacement, pins):
    monkeypatch.setattr(O, target, replacement)
    failed = False
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed = True
            break
    assert failed, f"planted mistake in {target} went unnoticed"


def test_mutation_swapped_nibbles(monkeypatch):
    _expect_pin_failure(monkeypatch, "pack_nibbles",
                        lambda c: (np.asarray(c)[:, 1::2] | (np.asarray(c)[:, 0::2] << 4)).astype(np.uint8),
                        [pin_nibble_layout])


def test_mutation_ties_away_from_zero(monkeypatch):
    def ties_up(lhs, mids, f):
        code = np.zeros(np.shape(lhs), dtype=np.int64)
        for u in mids:
            code += lhs >= u * f
        return code
    _expect_pin_failure(monkeypatch, "_nearest_code_ties_even", ties_up,
                        [lambda: pin_quantize_brute_force(tiny_inputs()[4])])


def test_mutation_ties_down(monkeypatch):
    def ties_down(lhs, mids, f):
        code = np.zeros(np.shape(lhs), dtype=np.int64)
        for u in mids:
            code += lhs > u * f
        return code
    _expect_pin_failure(monkeypatch, "_nearest_code_ties_even", ties_down,
                        [lambda: pin_quantize_brute_force(tiny_inputs()[4])])


def test_mutation_transposed_operand(monkeypatch):
    def linear_t(x_bits, packed, scales, tscale):
        x = O.bf16_to_f64(x_bits)
        w = O.dequant_exact(packed, scales, tscale)
        return x @ w, np.abs(x) @ np.abs(w)      # W not transposed (square case)
    w = WL.normal_bf16((16, 16), 0.02, 40)
    x = WL.normal_bf16((16, 16), 1.0, 41)
    _expect_pin_failure(monkeypatch, "linear_ref", linear_t,
                        [lambda: pin_linear_brute_force(x, *O.quantize(w))])


def test_mutation_dropped_tensor_scale(monkeypatch):
    orig = O.decoded_products
    w = WL.normal_bf16((4, 64), 0.02, 42)
    q = O.quantize(w)
    monkeypatch.setattr(O, "dequant", lambda p, s, t: O.f32_to_bf16_rne(orig(p, s).astype(np.float32)))
    with pytest.raises(AssertionError):
        pin_dequant_closed_form(*q)


def test_mutation_scale_from_rounded_tscale(monkeypatch):
    """Deciding codes against the rounded tscale instead of amax breaks exact ties."""
    orig = O.element_codes

    def via_tscale(w_bits, scale_codes, amax):
        t = float(O.tensor_scale(amax))
        return orig(w_bits, scale_codes, t * 2688.0 * (1 + 2 ** -22))
    _expect_pin_failure(monkeypatch, "element_codes", via_tscale,
                        [lambda: pin_quantize_brute_force(tiny_inputs()[4])])


def test_mutation_wrong_e4m3_bias(monkeypatch):
    bad = O.E4M3_TABLE * 2.0
    monkeypatch.setattr(O, "E4M3_TABLE", bad)
    with pytest.raises(AssertionError):
        pin_e4m3_table()


# --------------------------------------------------------------------------
# NVFP4 x NVFP4 linear (R20): activations quantized on the fly.
# --------------------------------------------------------------------------
def _brute_nvfp4_values(bits):
    """NVFP4 values of a BF16 matrix as Fractions, by exhaustive exact-rational nearest search
    (E4M3 grid from torch, E2M1 magnitudes from the page), one tensor scale for the whole matrix."""
    mags = [Fraction(v) for v in _read_golden("e2m1_magnitudes.txt")]
    rows = [[Fraction(float(a)) for a in row] for row in WL.f32_from_bf16_bits(bits)]
    amax = max(abs(a) for row in rows for a in row)
    if amax == 0:
        return [[Fraction(0)] * len(r) for r in rows]
    t = Fraction(float(np.float32(float(amax) / 2688.0)))
    out = []
    for row in rows:
        vals = []
        for b in range(0, len(row), 16):
            blk = row[b:b + 16]
            s = E4M3_GRID[_nearest_even(448 * max(abs(a) for a in blk) / amax, E4M3_GRID)]
            for a in blk:
                mag = 0 if s == 0 else mags[_nearest_even(2688 * abs(a) / (amax * s), mags)]
                vals.append((mag if a >= 0 else -mag) * s * t)
        out.append(vals)
    return out


def w4a4_inputs():
    rng = np.random.default_rng(60)
    x = rng.standard_normal((3, 48)) * np.array([[1.0], [0.07], [5.0]])   # rows of very different range
    x[0, 5] = 9.0                                                          # one outlier sets the tensor scale
    w = WL.normal_bf16((2, 48), 0.02, 61)
    return _bits(x), w


def pin_w4a4_brute_force():
    x_bits, w_bits = w4a4_inputs()
    packed, scales, tscale = O.quantize(w_bits)
    y_ref, bound = O.linear_w4a4_ref(x_bits, packed, scales, tscale)
    xv, wv = _brute_nvfp4_values(x_bits), _brute_nvfp4_values(w_bits)
    assert y_ref.shape == (len(xv), len(wv))
    for i in range(len(xv)):
        for j in range(len(wv)):
            exact = sum(a * b for a, b in zip(xv[i], wv[j]))
            babs = sum(abs(a * b) for a, b in zip(xv[i], wv[j]))
            tol = Fraction(1, 10 ** 12) * (babs + Fraction(1, 10 ** 30))
            assert abs(Fraction(y_ref[i, j]) - exact) <= tol, (i, j)
            assert abs(Fraction(bound[i, j]) - babs) <= tol, (i, j)


def test_w4a4_brute_force():
    pin_w4a4_brute_force()


def test_w4a4_on_grid_activations_reduce_to_w4a16():
    """X already on its own NVFP4 grid (a quantize-dequant fixed point) gives the weight-only result.

    amax = 10.5 = 2688 * 2^-8 makes the tensor scale a power of two, so the grid values are exact in BF16."""
    _, w_bits = w4a4_inputs()
    x = np.random.default_rng(62).standard_normal((3, 48))
    x[1, 7] = -10.5
    xp, xs, xt = O.quantize(_bits(x))
    assert float(xt) == 2.0 ** -8
    x_grid = O.dequant_exact(xp, xs, xt)
    xg_bits = O.f32_to_bf16_rne(x_grid.astype(np.float32))
    assert np.array_equal(O.bf16_to_f64(xg_bits), x_grid)
    q = O.quantize(w_bits)
    a, _ = O.linear_w4a4_ref(xg_bits, *q)
    b, _ = O.linear_ref(xg_bits, *q)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)


def test_mutation_w4a4_activations_not_quantized(monkeypatch):
    _expect_pin_failure(monkeypatch, "linear_w4a4_ref", lambda x, p, s, t: O.linear_ref(x, p, s, t),
                        [pin_w4a4_brute_force])


def test_mutation_w4a4_per_row_activation_scale(monkeypatch):
    def per_row(x_bits, packed, scales, tscale):
        rows = [O.quantize(x_bits[i:i + 1]) for i in range(x_bits.shape[0])]
        x = np.concatenate([O.dequant_exact(*r) for r in rows])
        w = O.dequant_exact(packed, scales, tscale)
        return x @ w.T, np.abs(x) @ np.abs(w).T
    _expect_pin_failure(monkeypatch, "linear_w4a4_ref", per_row, [pin_w4a4_brute_force])


def test_mutation_w4a4_weight_scale_for_activations(monkeypatch):
    def shared_scale(x_bits, packed, scales, tscale):
        xp, xs, _ = O.quantize(x_bits)
        x = O.dequant_exact(xp, xs, tscale)
        w = O.dequant_exact(packed, scales, tscale)
        return x @ w.T, np.abs(x) @ np.abs(w).T
    _expect_pin_failure(monkeypatch, "linear_w4a4_ref", shared_scale, [pin_w4a4_brute_force])


# --------------------------------------------------------------------------
# Expert stacks (R12, R13).
# --------------------------------------------------------------------------
def test_quantize_experts_one_tensor_scale_per_expert():
    """Each expert's tensor scale is fl32(its own amax / 2688); a shared amax would fail this."""
    w = np.stack([WL.normal_bf16((6, 48), 0.02 * 3.0 ** i, 40 + i) for i in range(3)])
    packed, scales, tscale = O.quantize_experts(w)
    assert packed.shape == (3, 6, 24) and scales.shape == (3, 6, 3) and tscale.shape == (3,)
    for i in range(3):
        amax = float(np.abs(WL.f32_from_bf16_bits(w[i])).max())
        assert tscale[i] == np.float32(amax) / np.float32(2688.0)
    assert len(set(tscale.tolist())) == 3
    pin_quantize_brute_force(w[1])
    p1, s1, _ = O.quantize(w[1])
    assert np.array_equal(packed[1], p1) and np.array_equal(scales[1], s1)
    d = O.dequant_experts(packed, scales, tscale)
    assert np.array_equal(d[2], O.dequant(packed[2], scales[2], tscale[2]))


def test_linear_routed_brute_force():
    """y[t, j, n] against an exact-rational sum over the expert chosen for (t, j), with duplicate and out-of-range ids."""
    mags = [Fraction(v) for v in _read_golden("e2m1_magnitudes.txt")]
    e2m1 = mags + [-m for m in mags]
    w = np.stack([WL.normal_bf16((4, 32), 0.02 * (i + 1), 60 + i) for i in range(3)])
    packed, scales, tscale = O.quantize_experts(w)
    x_bits = WL.normal_bf16((3, 32), 1.0, 70)
    route = np.array([[2, 0], [1, 1], [-1, 3]], dtype=np.int32)
    y, bound = O.linear_routed_ref(x_bits, route, packed, scales, tscale)
    assert y.shape == (3, 2, 4)
    x = WL.f32_from_bf16_bits(x_bits).astype(np.float64)
    for t in range(3):
        for j in range(2):
            e = int(route[t, j])
            for n in range(4):
                if not 0 <= e < 3:
                    assert y[t, j, n] == 0 and bound[t, j, n] == 0
                    continue
                codes = O.unpack_nibbles(packed[e])
                e4m3 = torch.from_numpy(scales[e].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                ts = Fraction(float(tscale[e]))
                terms = [Fraction(x[t, kk]) * e2m1[codes[n, kk]] * Fraction(e4m3[n, kk // 16]) * ts for kk in range(32)]
                exact, babs = sum(terms), sum(abs(v) for v in terms)
                tol = Fraction(1, 10 ** 12) * (babs + Fraction(1, 10 ** 30))
                assert abs(Fraction(y[t, j, n]) - exact) <= tol, (t, j, n)
                assert abs(Fraction(bound[t, j, n]) - babs) <= tol, (t, j, n)
    assert np.array_equal(y[1, 0], y[1, 1])  # the same expert twice


# ---------------------------------------------------------------------------
# FP4 KV-cache gather (oracle/kv_oracle.py).
# ---------------------------------------------------------------------------
from oracle import kv_oracle as KV  # noqa: E402


def test_ue8m0_table_matches_torch():
    """UE8M0 (OCP MX scale byte) against torch's float8_e8m0fnu cast, all 256 codes."""
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(KV.UE8M0_TABLE[255]) and np.isnan(t[255])
    assert np.array_equal(KV.UE8M0_TABLE[:255], t[:255])
    assert KV.UE8M0_TABLE[127] == 1.0 and KV.UE8M0_TABLE[0] == 2.0 ** -127 and KV.UE8M0_TABLE[254] == 2.0 ** 127


def _e2m1_signed(code, factor):
    """E2M1 nibble times a non-negative Fraction, as a float64 with the nibble's sign (code 0x8 is -0, so its
    products are -0): the bit layout written out, sign, exponent bias 1, one mantissa bit."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return math.copysign(float(mag * factor), -1.0 if s else 1.0)


def test_kv_decode_nvfp4_against_exact_products():
    """R15 (NVFP4): exact rational E2M1 * E4M3 * tscale, rounded once to float32 (exact in float64 first:
    at most 6 + 24 significant bits), then to FP16 / BF16 by torch's casts."""
    rng = np.random.default_rng(31)
    codes = rng.integers(0, 256, size=(6, 2, 16), dtype=np.uint8)       # 6 rows x 2 heads x 32 elements
    scales = rng.integers(0, 0x7F, size=(6, 2, 2), dtype=np.uint8)      # finite E4M3 codes
    scales[0, 0, 0], scales[1, 1, 1] = 0x7E, 0x01                        # 448 and the smallest subnormal
    ts = np.float32(0.0123)
    e4m3 = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    exact = np.empty((6, 2, 32), dtype=np.float64)                       # exact: <= 30 significant bits
    for idx in np.ndindex(6, 2):
        for d in range(32):
            byte = int(codes[idx][d // 2])
            nib = byte & 0xF if d % 2 == 0 else byte >> 4
            exact[idx + (d,)] = _e2m1_signed(nib, Fraction(float(e4m3[idx][d // 16])) * Fraction(float(ts)))
    f32 = torch.from_numpy(exact).to(torch.float32)
    for out, dt in ((KV.F16, torch.float16), (KV.BF16, torch.bfloat16)):
        want = f32.to(dt).view(torch.int16).numpy().view(np.uint16)
        got = KV.decode_rows(KV.NVFP4, out, codes, scales, ts)
        assert np.array_equal(got, want), out


def test_kv_decode_mxfp4_against_exact_products():
    """R15 (MXFP4): E2M1 * 2^(e - 127) exactly, one rounding to FP16 / BF16 (torch's casts from float64, exact
    through float32 for two significant bits), including FP16 overflow and underflow scales."""
    rng = np.random.default_rng(32)
    codes = rng.integers(0, 256, size=(5, 3, 32), dtype=np.uint8)       # 5 rows x 3 heads x 64 elements
    scales = rng.integers(90, 160, size=(5, 3, 2), dtype=np.uint8)
    scales[0, 0, 0], scales[0, 0, 1], scales[1, 0, 0], scales[1, 0, 1] = 0, 254, 140, 141
    for out, dt in ((KV.F16, torch.float16), (KV.BF16, torch.bfloat16)):
        want = np.empty((5, 3, 64), dtype=np.uint16)
        for idx in np.ndindex(5, 3):
            vals = []
            for d in range(64):
                byte = int(codes[idx][d // 2])
                nib = byte & 0xF if d % 2 == 0 else byte >> 4
                vals.append(_e2m1_signed(nib, Fraction(2) ** (int(scales[idx][d // 32]) - 127)))
            want[idx] = torch.tensor(vals, dtype=torch.float64).to(dt).view(torch.int16).numpy().view(np.uint16)
        got = KV.decode_rows(KV.MXFP4, out, codes, scales)
        assert np.array_equal(got, want), out
    # closed forms: scale 127 is the E2M1 table itself; FP16 overflows past 65504 (6 * 2^14 at e = 141)
    c = np.full((1, 16), 0x77, dtype=np.uint8)                             # 6.0 everywhere
    assert np.all(KV.decode_values(KV.MXFP4, c, np.array([[127]], dtype=np.uint8)) == 6.0)
    assert np.all(KV.decode_rows(KV.MXFP4, KV.F16, c, np.array([[140]], dtype=np.uint8)) == 0x7A00)   # 49152
    assert np.all(KV.decode_rows(KV.MXFP4, KV.F16, c, np.array([[141]], dtype=np.uint8)) == 0x7C00)   # +inf


def test_kv_gather_indexing_brute_force():
    """R16 on pages whose values name their source: every element of page p, slot i is 2^(p * 4 + i - 17)
    (MXFP4, codes 1.0, scale byte 110 + 4p + i), so each output row says which page and slot it came from."""
    nb, bs, heads, hd = 6, 4, 2, 32
    codes = np.full((nb, bs, heads, hd // 2), 0x22, dtype=np.uint8)      # E2M1 1.0 in both nibbles
    scales = np.empty((nb, bs, heads, 1), dtype=np.uint8)
    for p in range(nb):
        for i in range(bs):
            scales[p, i] = 110 + 4 * p + i
    block_table = np.array([[3, 0, 4, 5], [1, 7, 2, 0], [5, 2, 5, 1], [2, 2, 2, 2], [4, 3, 3, 3]], dtype=np.int32)
    seq_lens = np.array([10, 7, 40, 3, 5], dtype=np.int32)              # seq 2 asks for more than its 4 pages hold
    dst_start = np.array([1, 12, 20, -2, 38], dtype=np.int32)           # seq 3 starts before row 0, seq 4 runs past 39
    out_rows = 40
    sentinel = np.uint16(0x1234)
    init = np.full((out_rows, heads, hd), sentinel, dtype=np.uint16)
    # Expected sources, written out: (row, page, slot), rows that become zero; every other row is untouched.
    src = [(1 + i, 3, i) for i in range(4)] + [(5 + i, 0, i) for i in range(4)] + [(9, 4, 0), (10, 4, 1)]
    src += [(12 + i, 1, i) for i in range(4)]
    zero = [16, 17, 18]                                                  # seq 1, page id 7 (out of range)
    src += [(20 + i, 5, i) for i in range(4)] + [(24 + i, 2, i) for i in range(4)]
    src += [(28 + i, 5, i) for i in range(4)] + [(32 + i, 1, i) for i in range(4)]   # 16 tokens, no more
    src += [(0, 2, 2)]                                                   # seq 3: tokens 0, 1 fall before row 0
    src += [(38, 4, 0), (39, 4, 1)]                                      # seq 4: tokens 2..4 fall past row 39
    got = KV.kv_gather_ref(KV.MXFP4, KV.F16, codes, scales, None, block_table, seq_lens, dst_start, init)
    want = init.copy()
    for (r, p, i) in src:
        want[r] = np.float16(2.0 ** (4 * p + i - 17)).view(np.uint16)
    for r in zero:
        want[r] = 0
    assert np.array_equal(got, want)
    for r in (11, 19, 36, 37):                                           # gaps between sequences untouched
        assert np.all(got[r] == sentinel)


def _expect_kv_pin_failure(monkeypatch, target, replacement, pins):
    monkeypatch.setattr(KV, target, replacement)
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError):
            return
    raise AssertionError(f"planted mistake in kv_oracle.{target} went unnoticed")


KV_DECODE_PINS = [test_kv_decode_nvfp4_against_exact_products, test_kv_decode_mxfp4_against_exact_products]


def test_mutation_kv_swapped_nibbles(monkeypatch):
    def swapped(p):
        c = KV.unpack_nibbles.__wrapped__(p) if hasattr(KV.unpack_nibbles, "__wrapped__") else O.unpack_nibbles(p)
        out = c.copy()
        out[:, 0::2], out[:, 1::2] = c[:, 1::2], c[:, 0::2]
        return out
    _expect_kv_pin_failure(monkeypatch, "unpack_nibbles", swapped, KV_DECODE_PINS)


def test_mutation_kv_dropped_tensor_scale(monkeypatch):
    orig = KV.decode_values
    _expect_kv_pin_failure(monkeypatch, "decode_values",
                           lambda fmt, c, s, t=None: orig(fmt, c, s, None if fmt == KV.MXFP4 else 1.0), KV_DECODE_PINS)


def test_mutation_kv_mx_group_16(monkeypatch):
    _expect_kv_pin_failure(monkeypatch, "GROUP", {KV.NVFP4: 16, KV.MXFP4: 16}, KV_DECODE_PINS)


def test_mutation_kv_ue8m0_bias(monkeypatch):
    _expect_kv_pin_failure(monkeypatch, "UE8M0_TABLE", KV.UE8M0_TABLE * 2.0,
                           [test_ue8m0_table_matches_torch] + KV_DECODE_PINS)


def test_mutation_kv_rounding_toward_zero(monkeypatch):
    def rtz(values, out):
        v = np.asarray(values, dtype=np.float64)
        if out == KV.F16:
            r = v.astype(np.float16)
            over = np.abs(r.astype(np.float64)) > np.abs(v)
            r[over] = np.nextafter(r[over], np.float16(0))
            return r.view(np.uint16)
        b = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return b
    _expect_kv_pin_failure(monkeypatch, "round_out", rtz, KV_DECODE_PINS)


def test_mutation_kv_page_and_slot_swapped(monkeypatch):
    def buggy(fmt, out, codes, scales, tscale, block_table, seq_lens, dst_start, out_init):
        nb, bs = codes.shape[:2]
        y = np.array(out_init, dtype=np.uint16, copy=True)
        for s in range(block_table.shape[0]):
            n = min(max(int(seq_lens[s]), 0), block_table.shape[1] * bs)
            for i in range(n):
                row = int(dst_start[s]) + i
                if 0 <= row < y.shape[0]:
                    page = int(block_table[s, i % block_table.shape[1]])      # planted: wrong table index
                    y[row] = 0 if not 0 <= page < nb else KV.decode_rows(fmt, out, codes[page, i % bs],
                                                                          scales[page, i % bs], tscale)
        return y
    _expect_kv_pin_failure(monkeypatch, "kv_gather_ref", buggy, [test_kv_gather_indexing_brute_force])


def test_mutation_kv_length_not_clamped(monkeypatch):
    orig = KV.kv_gather_ref

    def unclamped(fmt, out, codes, scales, tscale, block_table, seq_lens, dst_start, out_init):
        # planted: tokens past the block table's capacity reuse its last page instead of being dropped
        cap = block_table.shape[1] * codes.shape[1]
        bt = np.concatenate([block_table, np.repeat(block_table[:, -1:], 8, axis=1)], axis=1)
        del cap
        return orig(fmt, out, codes, scales, tscale, bt, seq_lens, dst_start, out_init)
    _expect_kv_pin_failure(monkeypatch, "kv_gather_ref", unclamped, [test_kv_gather_indexing_brute_force])


# ---------------------------------------------------------------------------
# MXFP4 tensors and the W4A4 linear (oracle/mxfp4_oracle.py).
# ---------------------------------------------------------------------------
from oracle import mxfp4_oracle as MX  # noqa: E402

_E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
              Fraction(6)]


def _bf16_fraction(b):
    """A BF16 bit pattern as an exact Fraction (sign, 8-bit exponent bias 127, 7-bit mantissa, subnormals)."""
    s, e, m = (b >> 15) & 1, (b >> 7) & 0xFF, b & 0x7F
    v = Fraction(m, 128) * Fraction(2) ** -126 if e == 0 else (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return -v if s else v


def _mx_block_brute(bits):
    """R17 by brute force on exact rationals: floor(log2(amax)) by walking powers of two, each element by an
    exhaustive nearest search over the eight magnitudes (ties to the even code)."""
    vals = [_bf16_fraction(int(b)) for b in bits]
    amax = max(abs(v) for v in vals)
    if amax == 0:
        e = 0
    else:
        p = 0
        while Fraction(2) ** (p + 1) <= amax:
            p += 1
        while Fraction(2) ** p > amax:
            p -= 1
        e = min(max(p - 2 + 127, 0), 254)
    scale = Fraction(2) ** (e - 127)
    codes = []
    for b, v in zip(bits, vals):
        q = abs(v) / scale
        best = min(range(8), key=lambda c: (abs(q - _E2M1_MAGS[c]), c % 2))   # nearest, then the even code
        codes.append(((int(b) >> 15) << 3) | best)
    return e, codes


def pin_mx_quantizer_brute_force():
    rng = np.random.default_rng(41)
    rows = []
    for r in range(24):
        f = rng.standard_normal(64).astype(np.float32) * np.float32(2.0 ** rng.integers(-20, 20))
        rows.append(WL.bf16_bits_from_f32(f))
    w = np.stack(rows)
    w[0, :32] = 0                                            # an all-zero block
    w[1, 3] = 0x8000                                          # -0
    w[2, :32] = WL.bf16_bits_from_f32(np.full(32, 1e-39, dtype=np.float32))   # subnormal block: scale clamps at 0
    w[3, 32:] = WL.bf16_bits_from_f32(np.array([4, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, 6.5, 7.9, -5, -0.75] + [0] * 20,
                                               dtype=np.float32))                # midpoints and saturation
    packed, scales = MX.quantize(w)
    codes = O.unpack_nibbles(packed)
    for r in range(w.shape[0]):
        for b in range(2):
            e, cs = _mx_block_brute(w[r, 32 * b:32 * b + 32])
            assert scales[r, b] == e, (r, b)
            assert list(codes[r, 32 * b:32 * b + 32]) == cs, (r, b)


def pin_mx_closed_forms():
    # amax 4 -> floor(log2) 2 -> scale byte 127 (2^0); the midpoints go to the even codes, 6.5 and 7.9 saturate
    w = WL.bf16_bits_from_f32(np.array([[4, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, 6.5, 7.9, -5, -0.75] + [0] * 20],
                                       dtype=np.float32))
    packed, scales = MX.quantize(w)
    assert scales[0, 0] == 127
    assert list(O.unpack_nibbles(packed)[0, :12]) == [6, 0, 2, 2, 4, 4, 6, 6, 7, 7, 8 | 6, 8 | 2]
    # idempotence: the block maximum quantizes to 4 or 6 times the scale, so dequant -> quantize is the identity
    rng = np.random.default_rng(42)
    x = WL.bf16_bits_from_f32((rng.standard_normal((8, 96)) * 3).astype(np.float32))
    p1, s1 = MX.quantize(x)
    back = O.f32_to_bf16_rne(MX.dequant_exact(p1, s1).astype(np.float32))
    p2, s2 = MX.quantize(back)
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
    # every block's largest magnitude code is 6 or 7
    mags = O.unpack_nibbles(p1).reshape(8, 3, 32) & 7
    assert np.all(mags.max(axis=2) >= 6)


def pin_mx_linear():
    rng = np.random.default_rng(43)
    x = WL.bf16_bits_from_f32(rng.standard_normal((3, 64)).astype(np.float32))
    w = WL.bf16_bits_from_f32((rng.standard_normal((5, 64)) * 0.05).astype(np.float32))
    wp, ws = MX.quantize(w)
    y, bound = MX.linear_w4a4_ref(x, wp, ws)
    # exact rational sums of the brute-force-quantized operands
    def deq(bits):
        out = []
        for b in range(0, 64, 32):
            e, cs = _mx_block_brute(bits[b:b + 32])
            out += [(-1 if c & 8 else 1) * _E2M1_MAGS[c & 7] * Fraction(2) ** (e - 127) for c in cs]
        return out
    xq = [deq(x[i]) for i in range(3)]
    wq = [deq(w[j]) for j in range(5)]
    for i in range(3):
        for j in range(5):
            assert y[i, j] == float(sum(a * b for a, b in zip(xq[i], wq[j])))
            assert bound[i, j] == float(sum(abs(a * b) for a, b in zip(xq[i], wq[j])))
    # one-hot activation: X = e_7 quantizes exactly (amax 1 -> scale 2^-2, code 4), so Y is column 7 of W's values
    e7 = np.zeros((1, 64), dtype=np.uint16)
    e7[0, 7] = 0x3F80
    y1, _ = MX.linear_w4a4_ref(e7, wp, ws)
    assert np.array_equal(y1[0], MX.dequant_exact(wp, ws)[:, 7])


def test_mx_quantizer_brute_force():
    pin_mx_quantizer_brute_force()


def test_mx_closed_forms():
    pin_mx_closed_forms()


def test_mx_linear_exact():
    pin_mx_linear()


MX_PINS = [pin_mx_quantizer_brute_force, pin_mx_closed_forms, pin_mx_linear]


def _expect_mx_pin_failure(monkeypatch, target, replacement):
    monkeypatch.setattr(MX, target, replacement)
    for pin in MX_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            return
    raise AssertionError(f"planted mistake in mxfp4_oracle.{target} went unnoticed")


def test_mutation_mx_scale_exponent(monkeypatch):
    _expect_mx_pin_failure(monkeypatch, "E2M1_EMAX", 1)


def test_mutation_mx_block_16(monkeypatch):
    _expect_mx_pin_failure(monkeypatch, "MX_BLOCK", 16)


def test_mutation_mx_ties_up(monkeypatch):
    def ties_up(lhs, mids, rhs):
        return sum((lhs >= u * rhs).astype(np.int64) for u in mids)
    _expect_mx_pin_failure(monkeypatch, "_nearest_code_ties_even", ties_up)


def test_mutation_mx_transposed_linear(monkeypatch):
    orig = MX.dequant_exact

    def swapped_halves(p, s):
        v = orig(p, s)
        return np.concatenate([v[:, 32:], v[:, :32]], axis=1) if v.shape[1] >= 64 else v
    _expect_mx_pin_failure(monkeypatch, "dequant_exact", swapped_halves)


# ---------------------------------------------------------------------------
# The library's kernel-native layout (oracle/layout_oracle.py): pinned by the
# hand-derived positions of tests/golden/kernel_native_layout.txt, an
# element-level check of every nibble and scale, the round trip and padding.
# ---------------------------------------------------------------------------
from oracle import layout_oracle as LO  # noqa: E402


def _golden_layout_lines():
    path = os.path.join(os.path.dirname(__file__), "golden", "kernel_native_layout.txt")
    with open(path) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_kernel_native_layout_golden_positions():
    rng = np.random.default_rng(7100)
    packed = rng.integers(0, 256, size=(32, 128), dtype=np.uint8)
    scales = rng.integers(0, 127, size=(32, 16), dtype=np.uint8)
    prep = LO.prepare(packed, scales)
    assert prep.size == 4 * 1152
    lines = _golden_layout_lines()
    assert len(lines) == 24
    for ln in lines:
        if ln[0] == "packed":
            blk, slot, word = int(ln[1]), int(ln[2]), int(ln[3].rstrip(":"))
            row, src = int(ln[4]), [int(v) for v in ln[5:9]]
            off = blk * 1152 + 16 * slot + 4 * word
            assert list(prep[off:off + 4]) == list(packed[row, src]), ln
        else:
            blk, word = int(ln[1]), int(ln[2].rstrip(":"))
            row, src = int(ln[3]), [int(v) for v in ln[4:8]]
            off = blk * 1152 + 1024 + 4 * word
            assert list(prep[off:off + 4]) == list(scales[row, src]), ln


def test_kernel_native_layout_every_element_and_scale():
    """Each element k of row n sits in the block of tile n // 16 and quad k // 128 (block index
    quad * tiles + tile), slot 16 g + n % 16, word i, nibble e with k % 128 = 32 i + 8 g + e, and its scale in
    byte i of word 16 (g // 2) + n % 16 of the same block."""
    rng = np.random.default_rng(7101)
    n, k = 37, 384
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 127, size=(n, k // 16), dtype=np.uint8)
    prep = LO.prepare(packed, scales)
    codes = np.empty((n, k), dtype=np.uint8)
    codes[:, 0::2], codes[:, 1::2] = packed & 0xF, packed >> 4
    tiles = -(-n // 16)
    for row in range(n):
        t, r = divmod(row, 16)
        for kk in range(k):
            q, rem = divmod(kk, 128)
            i, rem = divmod(rem, 32)
            g, e = divmod(rem, 8)
            base = (q * tiles + t) * 1152
            byte = prep[base + 16 * (16 * g + r) + 4 * i + e // 2]
            assert ((byte >> (4 * (e % 2))) & 0xF) == codes[row, kk]
            assert prep[base + 1024 + 4 * (16 * (g // 2) + r) + i] == scales[row, kk // 16]


def test_kernel_native_layout_round_trip_and_padding():
    rng = np.random.default_rng(7102)
    for n, k in [(16, 128), (33, 256), (5, 640), (48, 128)]:
        packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        scales = rng.integers(0, 127, size=(n, k // 16), dtype=np.uint8)
        prep = LO.prepare(packed, scales)
        assert prep.size == LO.prepared_bytes(n, k) == -(-n // 16) * 16 * k * 9 // 16
        p2, s2 = LO.unprepare(prep, n, k)
        assert np.array_equal(p2, packed) and np.array_equal(s2, scales)
        assert LO.padding_is_zero(prep, n, k)
    with pytest.raises(ValueError):
        LO.prepared_bytes(16, 96)


def test_mutation_kernel_native_swapped_lane_groups(monkeypatch):
    """A planted mistake (slots of lane groups 1 and 2 exchanged) fails the golden positions."""
    orig = LO.prepare

    def bad(packed, scales):
        out = orig(packed, scales).copy()
        for blk in range(out.size // 1152):
            b = blk * 1152
            s1 = out[b + 256:b + 512].copy()
            out[b + 256:b + 512] = out[b + 512:b + 768]
            out[b + 512:b + 768] = s1
        return out

    monkeypatch.setattr(LO, "prepare", bad)
    with pytest.raises(AssertionError):
        test_kernel_native_layout_golden_positions()


def test_mutation_kernel_native_tile_major(monkeypatch):
    """A planted mistake (blocks in tile-major order, tile t's quads side by side) fails the golden positions."""
    orig = LO.prepare

    def bad(packed, scales):
        out = orig(packed, scales)
        n, k = packed.shape[0], 2 * packed.shape[1]
        tiles, quads = -(-n // 16), k // 128
        blocks = out.reshape(quads, tiles, 1152)          # quad-major as written
        return np.ascontiguousarray(blocks.transpose(1, 0, 2)).reshape(-1)

    monkeypatch.setattr(LO, "prepare", bad)
    with pytest.raises(AssertionError):
        test_kernel_native_layout_golden_positions()
