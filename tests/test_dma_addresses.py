"""CPU replay of the prefill GEMM's LDS-DMA source addresses (csrc/prefill.hip,
prefill_dma_kernel, dense form): for every workgroup, wavefront, load
instruction, lane and step -- including the loads issued past the last step,
which repeat the last step or group -- the 16 bytes each lane reads must lie
inside its buffer (x, packed or scales), the activation offsets must fit the
32-bit lane offsets the kernel uses, and every LDS destination must lie inside
its stage or group buffer.  The formulas are written out from the kernel's
source; no GPU is involved."""
import numpy as np
import pytest

BM, BN, BK, GK, WSLOTS = 128, 272, 64, 256, 9
LX, LW = 4, 10
WLAST = BN * WSLOTS - 64


def _cdiv(a, b):
    return -(-a // b)


def prefill_dma_check(m, n, k, clamp=True):
    assert k % GK == 0
    n_tiles, m_tiles = _cdiv(n, BN), _cdiv(m, BM)
    nsteps = k // BK
    kh, ks = k // 2, k // 16
    lane = np.arange(64)
    w = np.arange(4)[:, None]
    # Steps issued: 0..3 before the loop, then t + 4 for t < nsteps (up to nsteps + 3), clamped to nsteps - 1.
    tc = np.minimum(np.arange(nsteps + 4), nsteps - 1)
    gc = np.unique(tc >> 2)
    worst_x32 = 0
    for mt in range(m_tiles):
        m0 = mt * BM
        for i in range(LX):
            q = w + 4 * i
            r = 8 * q + (lane >> 3)                               # [4, 64]
            gm = np.where(m0 + r < m, r, m - 1 - m0) if clamp else r
            off = gm * k * 2 + 16 * ((lane & 7) ^ (r & 7))        # 32-bit lane offset from x + m0 k + tc * 128
            assert off.min() >= 0 and off.max() < 2 ** 32
            worst_x32 = max(worst_x32, int(off.max()))
            base = m0 * k * 2 + tc[:, None, None] * (2 * BK)
            addr = base + off[None]
            assert addr.min() >= 0 and (addr + 16).max() <= m * k * 2, (m, n, k, mt, i)
            dst = 1024 * (w + 4 * i) + 16 * lane                  # bytes into the 16 KiB X stage
            assert dst.min() >= 0 and (dst + 16).max() <= BM * 8 * 16
    for nt in range(n_tiles):
        n0 = nt * BN
        for i in range(LW):
            q0 = 64 * (w + 4 * i)
            qs = np.minimum(q0, WLAST)
            slot = qs + lane                                      # [4, 64]
            r, piece = slot // WSLOTS, slot % WSLOTS
            gn = np.where(n0 + r < n, n0 + r, n - 1) if clamp else n0 + r
            is_scale = piece == 8
            # Each instruction's scale lanes step 16 bytes per group, packed lanes 128.
            for g in gc:
                pa = gn * kh + 16 * piece + g * (GK // 2)
                sa = gn * ks + g * (GK // 16)
                assert (pa[~is_scale] >= 0).all() and (pa[~is_scale] + 16 <= n * kh).all(), (m, n, k, nt, i, g)
                assert (sa[is_scale] >= 0).all() and (sa[is_scale] + 16 <= n * ks).all(), (m, n, k, nt, i, g)
            dst = 16 * slot
            assert dst.min() >= 0 and (dst + 16).max() <= BN * WSLOTS * 16
    return worst_x32


# The down projection (N=5120, K=17408) and the prefill shape at the timed M, and the ragged test shapes.
SHAPES = [(512, 5120, 17408), (2048, 5120, 17408), (512, 17408, 5120), (2048, 17408, 5120),
          (200, 560, 768), (129, 545, 256), (300, 300, 2560), (130, 257, 2304), (65, 17, 256), (1, 1, 256)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_prefill_dma_sources_in_bounds(m, n, k):
    prefill_dma_check(m, n, k)


def test_prefill_dma_largest_supported_k_offsets_fit_32_bits():
    # prefill_dma_supported admits k < 2^24: the largest activation lane offset must still fit 32 bits.
    k = (1 << 24) - GK
    r = 127
    assert r * k * 2 + 16 * 7 < 2 ** 32


def test_replay_catches_a_planted_overrun():
    # The checker itself: without the kernel's clamps of rows past m and n, a ragged tile reads past the end.
    with pytest.raises(AssertionError):
        prefill_dma_check(129, 545, 256, clamp=False)
    prefill_dma_check(129, 545, 256, clamp=True)


# ---------------------------------------------------------------------------
# The launch's tile mapping with split tiles (csrc/prefill.hip, prefill_split and
# the head of prefill_dma_kernel), written out: every output tile is computed
# over the whole K exactly once (whole, or as slices that partition its K
# groups), and every split tile's slot and counter indices stay inside the
# workspace the plan sizes.
# ---------------------------------------------------------------------------
def prefill_split_plan(m, n, k):
    tiles = _cdiv(n, BN) * _cdiv(m, BM)
    groups = k // GK
    r = tiles % 256
    if tiles <= 128:
        dp, c = 0, min(4, 256 // tiles)
    elif tiles > 256 and 0 < r <= 128:
        dp, c = tiles - r, min(8, 256 // r)
    else:
        return None
    c = min(c, groups)
    if c < 2:
        return None
    return dp, tiles - dp, c


def _remap(b, n):
    return (b & 7) * (n >> 3) + (b >> 3) if n % 8 == 0 else b


def prefill_split_cover(m, n, k):
    tiles, groups = _cdiv(n, BN) * _cdiv(m, BM), k // GK
    dp, tail, c = prefill_split_plan(m, n, k)
    grid = dp + tail * c
    cover = np.zeros((tiles, groups), dtype=np.int64)
    slots = set()
    for b in range(grid):
        if b < dp:
            cover[_remap(b, dp), :] += 1
            continue
        j = _remap(b - dp, grid - dp)
        xt, sl = j // c, j % c
        g0, g1 = sl * groups // c, (sl + 1) * groups // c
        assert 0 <= xt < tail and 0 <= sl < c and g1 > g0
        cover[dp + xt, g0:g1] += 1
        assert (xt, sl) not in slots
        slots.add((xt, sl))
        assert 4 * xt + 4 <= 16384                                  # counter inside the counter region
        assert (xt * c + sl + 1) * 139264 <= tail * c * 139264      # partial tile inside the workspace
    assert (cover == 1).all(), (m, n, k)
    return dp, tail, c


@pytest.mark.parametrize("m,n,k", [(2048, 5120, 17408), (512, 5120, 17408), (65, 17408, 5120), (200, 560, 768),
                                   (129, 545, 256 * 3), (4000, 2200, 512), (2049, 5120, 1024), (3500, 5120, 2048),
                                   (4200, 5120, 512), (8192, 5120, 17408)])
def test_prefill_split_tiles_cover_k_once(m, n, k):
    plan = prefill_split_plan(m, n, k)
    if plan is None:
        pytest.skip("no split for this shape")
    prefill_split_cover(m, n, k)


def test_prefill_split_plan_shapes():
    assert prefill_split_plan(2048, 5120, 17408) == (256, 48, 5)    # 304 tiles
    assert prefill_split_plan(512, 5120, 17408) == (0, 76, 3)
    assert prefill_split_plan(512, 17408, 5120) is None             # 256 tiles fill a round
    assert prefill_split_plan(2048, 17408, 5120) is None            # 1024 tiles
    assert prefill_split_plan(8192, 5120, 17408) is None            # 1216 tiles: 4 rounds and 192 more
    assert prefill_split_plan(3500, 5120, 2048) == (512, 20, 8)     # 532 tiles: 2 rounds and 20 more
    assert prefill_split_plan(4200, 5120, 512) == (512, 115, 2)     # 627 tiles: 2 rounds and 115 more


# ---------------------------------------------------------------------------
# Small-M kernel with activations staged through LDS (csrc/small_m.hip,
# small_m_xl_kernel): each wavefront copies a quad's MX activation rows x 256
# bytes into its own LDS area, instruction d and lane l covering row
# r = 4 d + l / 16 (rows past m repeat row m - 1) at slot l % 16, which holds
# the row's 16-byte piece (l % 16) ^ (r % 16); the fragment read of step i,
# m tile mt by lane (c, g) = (l % 16, l / 16) takes row rr = min(16 mt + c,
# m - 1) at slot (4 i + g) ^ (rr % 16).
# ---------------------------------------------------------------------------
SM_QUAD_K = 128


def small_m_xl_check(m, k, mx):
    """Replays one wavefront's copies and fragment reads for every quad: every copy source lies inside x [m, k],
    every LDS byte written or read lies inside the wavefront's quad area, and each fragment read finds exactly
    the 8 activations x[row, 128 q + 32 i + 8 g, + 8) that the MFMA step expects."""
    assert 1 <= m <= mx and mx in (8, 16, 32) and k % SM_QUAD_K == 0
    D, XB = mx // 4, mx * 256
    nmt = (mx + 15) // 16
    lane = np.arange(64)
    quads = k // SM_QUAD_K
    for q in range(quads):
        area = {}                               # LDS byte offset in the area -> global element index
        for d in range(D):
            r = 4 * d + (lane >> 4)
            gr = np.minimum(r, m - 1)
            piece = (lane & 15) ^ (r & 15)
            src = gr * k + 8 * piece + q * SM_QUAD_K          # element index of the lane's 16 bytes
            assert src.min() >= 0 and (src + 8).max() <= m * k
            dst = d * 1024 + 16 * lane
            assert dst.min() >= 0 and (dst + 16).max() <= XB
            for l in range(64):
                area[int(dst[l])] = int(src[l])
        for mt in range(nmt):
            rr = np.minimum(16 * mt + (lane & 15), m - 1)
            for i in range(4):
                g = lane >> 4
                off = rr * 256 + ((4 * i + g) ^ (rr & 15)) * 16
                assert off.min() >= 0 and (off + 16).max() <= XB
                want = rr * k + q * SM_QUAD_K + 32 * i + 8 * g
                got = np.array([area[int(o)] for o in off])
                assert np.array_equal(got, want)


@pytest.mark.parametrize("mx", [8, 16, 32])
def test_small_m_xl_copies_and_reads(mx):
    lo = {8: 1, 16: 9, 32: 17}[mx]
    for m in sorted({lo, lo + 1, (lo + mx) // 2, mx - 1, mx}):
        for k in (128, 384, 5120):
            small_m_xl_check(m, k, mx)


def test_small_m_xl_reads_hit_distinct_bank_groups():
    """The 16 lanes of a fragment read that share g read 16 different rows at 16 different 16-byte slots of
    their 256-byte rows: one pass of the LDS banks, no conflict."""
    lane = np.arange(16)
    for mt in range(2):
        rr = 16 * mt + lane
        for i in range(4):
            for g in range(4):
                slot = (4 * i + g) ^ (rr & 15)
                assert len(set(slot.tolist())) == 16


def test_splitk_partial_slots_are_a_permutation():
    """The split-K partial-sum layout (csrc/device_common.hpp, splitk_store_rows4): the 4-row group at n0 of an
    activation row keeps its four values at slots s + 2j, s + 2j + 1, s + 8 + 2j, s + 9 + 2j, with s = n0 & ~15
    and j = (n0 / 4) % 4; over every group of a row padded to a multiple of 16 the slots are each used once, and a
    store instruction's four groups of one span write the two 32-byte halves of the span."""
    for npad in (16, 32, 5120, 13664):
        slots = []
        for n0 in range(0, npad, 4):
            s, j = n0 & ~15, (n0 >> 2) & 3
            slots += [s + 2 * j, s + 2 * j + 1, s + 8 + 2 * j, s + 9 + 2 * j]
        assert sorted(slots) == list(range(npad))
    first = sorted(s for n0 in range(0, 16, 4) for s in ((n0 & ~15) + 2 * ((n0 >> 2) & 3),
                                                         (n0 & ~15) + 2 * ((n0 >> 2) & 3) + 1))
    assert first == list(range(8))
