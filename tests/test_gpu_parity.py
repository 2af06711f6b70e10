"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Quantize and dequant must match bit for bit; the linear must satisfy
|y - y_ref| <= 2e-3 * sum_k |x * w_hat| per output element (y_ref exact in
float64).  Small and ragged shapes are checked in full; the full-size
workloads are checked on sampled weight rows / output columns, in the launch
configuration the benchmark times (auto dispatch).
"""
import sys
import time

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from nvfp4_weight_only_amd import workloads as WL

pytestmark = pytest.mark.gpu

KERNELS = ["gemv", "small_m", "prefill"]


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_weight_only_amd as nv
    nv.lib()   # fails loudly when the library is missing
    return nv


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def bf16_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8_host(t):
    return t.cpu().numpy()


def sample_rows(n, count, seed=123):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(count, n), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(rows))


def q_both(nv, w_bits):
    """w quantized on the GPU (device tensors) and by the oracle (host arrays), checked bit-equal.

    The oracle's linear always runs on the oracle's own quantization, never on
    the GPU's outputs."""
    q = nv.quantize(to_dev_bf16(w_bits))
    rp, rs, rt = O.quantize(w_bits)
    assert np.array_equal(u8_host(q[0]), rp) and np.array_equal(u8_host(q[1]), rs), "quantization differs"
    assert q[2].cpu().numpy()[0].view(np.uint32) == np.float32(rt).view(np.uint32), "tensor scale differs"
    return q, (rp, rs, rt)


def check_linear(y_bits, y_ref, bound, what):
    y = WL.f32_from_bf16_bits(y_bits).astype(np.float64)
    bad = O.linear_violations(y, y_ref, bound)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(bound > 0, np.abs(y - y_ref) / bound, 0.0)
    log(f"{what}: max |y-y_ref|/B = {rel.max():.3e}, median {np.median(rel):.3e}")
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside 2e-3*B (max rel {rel.max():.3e})"
    return rel


# ---------------------------------------------------------------------------
# Quantize / dequant, small and ragged shapes, bit-exact.
# ---------------------------------------------------------------------------
SMALL_WEIGHTS = [
    ("tiny 256x512", lambda: WL.weight_plain(256, 512)),
    ("ragged 300x1040", lambda: WL.normal_bf16((300, 1040), 0.02, 5)),   # k % 32 == 16
    ("ragged 77x48", lambda: WL.normal_bf16((77, 48), 0.02, 6)),
    ("one block 1x16", lambda: WL.normal_bf16((1, 16), 0.02, 7)),
    ("outliers 64x5120", lambda: WL.weight_with_outlier_columns(64, 5120)),
    ("wide range 33x272", lambda: WL.bf16_bits_from_f32(
        (np.random.default_rng(8).standard_normal((33, 272)) *
         np.exp(np.random.default_rng(9).uniform(-30, 30, (33, 272)))).astype(np.float32))),
]


def crafted_weights():
    """Ties on every E2M1 and E4M3 midpoint, zeros, -0, BF16 subnormals, huge values."""
    row = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -0.0]
    row2 = [3.0, 0.125, 0.375, 0.625, 0.875, 1.25, 1.75, 2.5, 0.0, -0.0, 1e-30, -1e-30, 2.0, 0.1, 0.2, 0.3]
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = (e4[:-1] + e4[1:]) / 2
    blocks = []
    for u in mids:
        blk = [0.0] * 16
        blk[3] = u
        blk[9] = -u / 3
        blocks.append(blk)
    cases = {
        "e2m1 ties": [row + row2],
        "e4m3 ties": [sum(blocks[i:i + 2], []) + [448.0] + [0.0] * 15 for i in range(0, 126, 2)],
        "zeros": [[0.0] * 31 + [-0.0]],
        "single": [[0.0] * 7 + [-0.0371] + [0.0] * 24],
        "subnormal amax": [[1e-40, -2e-39, 3e-41, 0.0] * 8],
        "huge": [[3.0e38, -1.0e38, 1.0, -1e-30] * 8],
        "far blocks": [[100.0] + [0.0] * 15 + [1e-3] + [0.0] * 15 + [1e-7] + [0.0] * 15],
    }
    return {k: WL.bf16_bits_from_f32(np.array(v, dtype=np.float32)) for k, v in cases.items()}


def _quant_compare(nv, w_bits, what):
    wd = to_dev_bf16(w_bits)
    packed, scales, tscale = nv.quantize(wd)                     # nvfp4_quantize_ws (two launches)
    p3, s3, t3 = nv.quantize(wd, workspace=None)                 # nvfp4_quantize (three launches)
    assert torch.equal(p3, packed) and torch.equal(s3, scales) and torch.equal(t3, tscale), \
        f"{what}: the two quantizer forms differ"
    rp, rs, rt = O.quantize(w_bits)
    gp, gs, gt = u8_host(packed), u8_host(scales), tscale.cpu().numpy()[0]
    assert gt.view(np.uint32) == np.float32(rt).view(np.uint32), f"{what}: tscale {gt} vs {rt}"
    assert np.array_equal(gs, rs), f"{what}: {int((gs != rs).sum())} scale codes differ"
    assert np.array_equal(gp, rp), f"{what}: {int((gp != rp).sum())} packed bytes differ"
    dq = bf16_host(nv.dequant(packed, scales, tscale))
    assert np.array_equal(dq, O.dequant(rp, rs, rt)), f"{what}: dequant differs"
    return packed, scales, tscale


@pytest.mark.parametrize("name,make", SMALL_WEIGHTS, ids=[s[0] for s in SMALL_WEIGHTS])
def test_quantize_dequant_bit_exact_small(nv, name, make):
    log(f"quantize/dequant {name}")
    _quant_compare(nv, make(), name)


def test_quantize_dequant_bit_exact_crafted(nv):
    for name, w in crafted_weights().items():
        log(f"quantize/dequant crafted: {name}")
        _quant_compare(nv, w, name)


def test_quantize_ws_ignores_workspace_contents(nv):
    """nvfp4_quantize_ws writes its partial maxima before reading them: a workspace full of 0xFF bytes (and one
    holding a previous call's maxima of a larger tensor) gives the same bits as the three-launch form."""
    w_big = WL.normal_bf16((1000, 4096), 0.5, 8101)
    w = WL.normal_bf16((300, 1040), 0.02, 8102)
    ws = torch.full((nv.lib().nvfp4_quantize_workspace_bytes(),), 0xFF, dtype=torch.uint8, device="cuda")
    for src in (w, w_big, w):
        wd = to_dev_bf16(src)
        a = nv.quantize(wd, workspace=ws)
        b = nv.quantize(wd, workspace=None)
        assert all(torch.equal(u, v) for u, v in zip(a, b))


@pytest.mark.parametrize("n,k", [(4096, 4096), (4353, 4096), (5120, 5120)])
def test_quantize_ws_amax_at_either_end(nv, n, k):
    """The amax pass of nvfp4_quantize_ws sees the first and the last element: a spike placed at either end sets
    the tensor scale.  4096 x 4096 fills its 1,024 workgroups' loads exactly once; the two larger shapes take a
    second, partial pass (4353 x 4096: its last load vector ends inside a workgroup's share)."""
    base = WL.weight_plain(n, k)
    for where, val in (((n - 1, k - 1), 300.0), ((0, 0), -400.0)):
        w = base.copy()
        w[where] = WL.bf16_bits_from_f32(np.array([val], dtype=np.float32))[0]
        log(f"quantize_ws amax spike {val} at {where}, {n}x{k}")
        _, _, tscale = nv.quantize(to_dev_bf16(w))
        want = O.tensor_scale(O.tensor_amax(w))
        assert float(O.tensor_amax(w)) == abs(val)
        assert tscale.cpu().numpy()[0].view(np.uint32) == np.float32(want).view(np.uint32)


def test_quantize_then_split_linear_share_a_stream(nv):
    """The binding's quantizer and split-K linear workspaces on one stream: a quantize between two split-K calls
    leaves the second one's arrival counters at zero (it has its own buffer), so both calls give the same bits as
    a call on a fresh zeroed workspace."""
    m, n, k = 8, 512, 17408
    w = WL.normal_bf16((n, k), 0.02, 8103)
    x = to_dev_bf16(WL.normal_bf16((m, k), 1.0, 8104))
    packed, scales, tscale = nv.quantize(to_dev_bf16(w))
    need = nv.lib().nvfp4_linear_workspace_bytes(m, n, k)
    assert need > 0, "this shape splits K"
    fresh = torch.zeros(need, dtype=torch.uint8, device="cuda")
    want = bf16_host(nv.linear(x, packed, scales, tscale, workspace=fresh))
    y1 = bf16_host(nv.linear(x, packed, scales, tscale))
    nv.quantize(to_dev_bf16(WL.normal_bf16((64, 4096), 1.0, 8105)))
    y2 = bf16_host(nv.linear(x, packed, scales, tscale))
    assert np.array_equal(y1, want) and np.array_equal(y2, want)


def test_quantize_crafted_ties_tiled(nv):
    """The crafted tie rows tiled to 640 x 1024, so that most blocks take the quantize kernel's whole-iteration
    path (the small crafted cases above take only its guarded tail); also as NVFP4 x NVFP4 activations, with
    the decoded BF16 values checked bit for bit."""
    cw = crafted_weights()
    for name, reps in (("e2m1 ties", (640, 32)), ("e4m3 ties", (10, 32))):
        w = np.ascontiguousarray(np.tile(cw[name], reps))
        log(f"quantize/dequant tiled {name}: {w.shape}")
        _quant_compare(nv, w, f"tiled {name}")
    x = np.ascontiguousarray(np.tile(cw["e2m1 ties"], (640, 32)))
    m, k = x.shape
    wq = WL.normal_bf16((48, k), 0.02, 3970)
    (packed, scales, tscale), (rp, rs, rt) = q_both(nv, wq)
    ws = torch.empty(nv.linear_w4a4_workspace_bytes(m, k), dtype=torch.uint8, device="cuda")
    y = bf16_host(nv.linear_w4a4(to_dev_bf16(x), packed, scales, tscale, workspace=ws))
    _w4a4_workspace_check(ws, x, m, k, rt)
    y_ref, bound = O.linear_w4a4_ref(x, rp, rs, rt)
    check_linear(y, y_ref, bound, "nvfp4 w4a4 tiled ties")


# ---------------------------------------------------------------------------
# Full-size weights: exact on sampled rows (the quantizer is row-local once amax is known).
# ---------------------------------------------------------------------------
FULL = ["decode", "gate_up", "small_m_up", "small_m_down"]


@pytest.mark.parametrize("wname", FULL)
def test_quantize_dequant_bit_exact_full_size(nv, wname):
    wl = WL.WORKLOADS[wname]
    log(f"full-size quantize {wname}: {wl.n}x{wl.k}")
    w = wl.weight()
    packed, scales, tscale = nv.quantize(to_dev_bf16(w))
    amax = O.tensor_amax(w)
    assert tscale.cpu().numpy()[0].view(np.uint32) == O.tensor_scale(amax).view(np.uint32)
    rows = sample_rows(wl.n, 96)
    rp, rs, rt = O.quantize(w[rows], amax=amax)
    rows_t = torch.from_numpy(rows).cuda()
    gp = u8_host(packed.index_select(0, rows_t))
    gs = u8_host(scales.index_select(0, rows_t))
    assert np.array_equal(gs, rs), f"{int((gs != rs).sum())} scale codes differ"
    assert np.array_equal(gp, rp), f"{int((gp != rp).sum())} packed bytes differ"
    dq = nv.dequant(packed, scales, tscale)
    assert np.array_equal(bf16_host(dq.index_select(0, rows_t)), O.dequant(rp, rs, rt))


def test_gate_up_shared_scale(nv):
    """Members quantized separately against a shared amax equal the merged quantization."""
    wl = WL.WORKLOADS["gate_up"]
    gate, up, ratio = WL.weight_gate_up(wl.n // 2, wl.k)
    log(f"gate/up amax ratio {ratio:.4f}")
    merged = nv.quantize(to_dev_bf16(np.concatenate([gate, up])))
    (pg, sg), (pu, su) = nv.quantize_shared([to_dev_bf16(gate), to_dev_bf16(up)])[0]
    _, ts = nv.quantize_shared([to_dev_bf16(gate), to_dev_bf16(up)])
    assert torch.equal(torch.cat([pg, pu]), merged[0])
    assert torch.equal(torch.cat([sg, su]), merged[1])
    assert torch.equal(ts, merged[2])
    # Wrong-scale failure mode: U decoded against its own tensor scale.
    own = nv.quantize(to_dev_bf16(up))[2]
    x = WL.activations(1, wl.k)
    y_right = bf16_host(nv.linear(to_dev_bf16(x), pu, su, ts))
    y_wrong = bf16_host(nv.linear(to_dev_bf16(x), pu, su, own))
    rows = sample_rows(wl.n // 2, 64)
    shared = max(O.tensor_amax(gate), O.tensor_amax(up))
    rp, rs, rt = O.quantize(up[rows], amax=shared)
    assert np.array_equal(u8_host(pu)[rows], rp) and np.array_equal(u8_host(su)[rows], rs)
    assert ts.cpu().numpy()[0].view(np.uint32) == O.tensor_scale(shared).view(np.uint32)
    y_ref, bound = O.linear_ref(x, rp, rs, rt)
    check_linear(y_right[:, rows], y_ref, bound, "gate/up shared scale (up rows)")
    # U's own scale is smaller by the amax spread: outputs shrink by that factor, and every output
    # whose |y| is not tiny against its bound falls outside the tolerance.
    yw = WL.f32_from_bf16_bits(y_wrong[:, rows]).astype(np.float64)
    bad = O.linear_violations(yw, y_ref, bound)
    big = np.abs(y_ref) > 0.01 * bound
    assert big.sum() > 20 and bad[big].all()
    shrink = np.median(np.abs(y_ref[big]) / np.abs(yw[big]))
    assert abs(shrink - ratio) / ratio < 0.02, shrink


# ---------------------------------------------------------------------------
# Linear: every kernel on small / ragged shapes, in full.
# ---------------------------------------------------------------------------
LIN_SHAPES = [(1, 256, 512), (3, 300, 1040), (8, 77, 48), (17, 130, 272), (32, 64, 5120), (33, 200, 512),
              (100, 300, 1040), (130, 257, 2064), (1, 1, 16), (5, 3, 16),
              # GEMV dispatch branches.  K split across wavefronts (k a multiple of 512 up to 5120):
              # 2, 6 and 9 wavefronts, ragged last 20-row workgroup, many workgroups.  Long K (a multiple of
              # 512 above 5120) on 16 wavefronts: 11 slices (five wavefronts without one), 12 slices, many
              # workgroups, 34 slices (two or three per wavefront) and 64 (four each).  LDS-staged rows:
              # ragged 64 lanes/row (k = 1056, 4640).  Neither (k = 5200)
              (1, 100, 1024), (2, 70, 3072), (1, 33, 4608), (1, 16500, 1024), (3, 300, 5632), (2, 70, 6144),
              (1, 100, 1056), (1, 33, 4640), (1, 16400, 6144), (1, 40, 17408), (1, 37, 32768), (1, 50, 5200),
              # prefill with K a multiple of 256: several 128 x 272 tiles with ragged edges, one K group
              (200, 560, 768), (129, 545, 256), (300, 300, 2560),
              # more small-M shapes: k = 128 and 384, 4-row workgroups, ragged n with two m tiles, large n
              (2, 100, 128), (5, 1000, 384), (31, 77, 640), (8, 10240, 512), (17, 4352, 256)]


@pytest.mark.parametrize("m,n,k", LIN_SHAPES)
def test_linear_all_kernels_small(nv, m, n, k):
    w = WL.normal_bf16((n, k), 0.02, 100 + n)
    x = WL.normal_bf16((m, k), 1.0, 200 + m)
    (packed, scales, tscale), rq = q_both(nv, w)
    y_ref, bound = O.linear_ref(x, *rq)
    xd = to_dev_bf16(x)
    outs = {}
    for kern in ["auto"] + KERNELS:
        y = bf16_host(nv.linear(xd, packed, scales, tscale, kernel=kern))
        check_linear(y, y_ref, bound, f"linear {kern} m={m} n={n} k={k}")
        outs[kern] = y
    # Deterministic: a second call is bitwise identical.
    for kern in KERNELS:
        assert np.array_equal(bf16_host(nv.linear(xd, packed, scales, tscale, kernel=kern)), outs[kern])


def test_linear_edge_cases(nv):
    # m = 0: a no-op
    packed, scales, tscale = nv.quantize(to_dev_bf16(WL.normal_bf16((64, 64), 0.02, 1)))
    y = nv.linear(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), packed, scales, tscale)
    assert y.shape == (0, 64)
    # zero weights and zero activations give exact zeros
    zw = nv.quantize(torch.zeros((48, 96), dtype=torch.bfloat16, device="cuda"))
    x = to_dev_bf16(WL.normal_bf16((5, 96), 1.0, 2))
    rw = nv.quantize(to_dev_bf16(WL.normal_bf16((48, 96), 0.02, 4)))
    for kern in KERNELS:
        assert torch.count_nonzero(nv.linear(x, *zw, kernel=kern)) == 0
        assert torch.count_nonzero(nv.linear(torch.zeros_like(x), *rw, kernel=kern)) == 0
    # crafted weights through every kernel
    for name, w in crafted_weights().items():
        if name in ("huge", "subnormal amax"):
            continue   # outputs overflow / underflow BF16 by construction
        q, rq = q_both(nv, w)
        x = WL.normal_bf16((3, w.shape[1]), 1.0, 3)
        y_ref, bound = O.linear_ref(x, *rq)
        for kern in KERNELS:
            check_linear(bf16_host(nv.linear(to_dev_bf16(x), *q, kernel=kern)), y_ref, bound, f"crafted {name} {kern}")


# ---------------------------------------------------------------------------
# Small-M kernel with K split across workgroups (caller workspace).
# ---------------------------------------------------------------------------
SPLIT_SHAPES = [(8, 300, 1040), (17, 130, 272), (32, 64, 5120), (33, 200, 512), (64, 5120, 5120), (16, 33, 4608),
                (64, 257, 2064), (9, 513, 784), (2, 5120, 2048), (24, 700, 3072), (3, 2000, 8192)]


@pytest.mark.parametrize("m,n,k", SPLIT_SHAPES)
def test_small_m_split_k(nv, m, n, k):
    need = nv.linear_workspace_bytes(m, n, k)
    assert need > 0, "shape expected to split K"
    w = WL.normal_bf16((n, k), 0.02, 300 + n)
    x = WL.normal_bf16((m, k), 1.0, 400 + m)
    q, rq = q_both(nv, w)
    y_ref, bound = O.linear_ref(x, *rq)
    xd = to_dev_bf16(x)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y1 = bf16_host(nv.linear(xd, *q, workspace=ws))
    check_linear(y1, y_ref, bound, f"split-K m={m} n={n} k={k}")
    # The arrival counters are back at zero: a second call on the same workspace
    # gives the same bits (a stale counter would leave output rows unwritten).
    for _ in range(2):
        assert np.array_equal(bf16_host(nv.linear(xd, *q, workspace=ws)), y1)
    # Unsplit, and a too-small workspace (which runs the unsplit kernel).
    y0 = bf16_host(nv.linear(xd, *q, workspace=None))
    check_linear(y0, y_ref, bound, f"unsplit m={m} n={n} k={k}")
    assert np.array_equal(bf16_host(nv.linear(xd, *q, workspace=ws[:need - 16])), y0)


def test_small_m_workspace_shared_by_shapes(nv):
    # One workspace, large enough for both, used alternately by two shapes.
    shapes = [(8, 300, 1040), (32, 5120, 2048)]
    ws = torch.zeros(max(nv.linear_workspace_bytes(*s) for s in shapes), dtype=torch.uint8, device="cuda")
    cases = []
    for i, (m, n, k) in enumerate(shapes):
        q, rq = q_both(nv, WL.normal_bf16((n, k), 0.02, 500 + i))
        x = WL.normal_bf16((m, k), 1.0, 600 + i)
        cases.append((to_dev_bf16(x), q, O.linear_ref(x, *rq)))
    for _ in range(3):
        for xd, q, (y_ref, bound) in cases:
            check_linear(bf16_host(nv.linear(xd, *q, workspace=ws)), y_ref, bound, "shared workspace")


# ---------------------------------------------------------------------------
# Linear at full size, auto dispatch, sampled output columns.
# ---------------------------------------------------------------------------
FULL_LINEAR = [("decode", 1), ("gate_up", 1), ("small_m_down", 1), ("small_m_up", 8), ("small_m_up", 32),
               ("small_m_down", 8),
               ("small_m_down", 32), ("prefill", 512), ("prefill", 2048), ("small_m_down", 512),
               ("prefill_down", 2048), ("prefill", 128)]

_weights_cache = {}


def _quantized(nv, wname):
    """(device quantization, BF16 weight, tensor amax) of a full-size workload weight."""
    if wname not in _weights_cache:
        _weights_cache.clear()
        # the prefill workloads share the small-M weights (same shapes and recipe)
        w = WL.WORKLOADS[{"prefill": "small_m_up", "prefill_down": "small_m_down"}.get(wname, wname)].weight()
        _weights_cache[wname] = (nv.quantize(to_dev_bf16(w)), w, O.tensor_amax(w))
    return _weights_cache[wname]


@pytest.mark.parametrize("wname,m", FULL_LINEAR, ids=[f"{a}-m{b}" for a, b in FULL_LINEAR])
def test_linear_full_size_sampled(nv, wname, m):
    wl = WL.WORKLOADS[wname]
    log(f"full-size linear {wname} m={m} n={wl.n} k={wl.k}")
    (packed, scales, tscale), w, amax = _quantized(nv, wname)
    x = WL.activations(m, wl.k)
    xd = to_dev_bf16(x)
    y = nv.linear(xd, packed, scales, tscale)
    y2 = nv.linear(xd, packed, scales, tscale)
    assert torch.equal(y, y2), "not deterministic"
    cols = sample_rows(wl.n, 64)
    cols_t = torch.from_numpy(cols).cuda()
    # The oracle quantizes the sampled rows itself (against the full tensor's amax); they must
    # equal the GPU's rows, and the oracle's linear runs on its own quantization.
    rp, rs, rt = O.quantize(w[cols], amax=amax)
    assert np.array_equal(u8_host(packed.index_select(0, cols_t)), rp)
    assert np.array_equal(u8_host(scales.index_select(0, cols_t)), rs)
    assert tscale.cpu().numpy()[0].view(np.uint32) == np.float32(rt).view(np.uint32)
    y_ref, bound = O.linear_ref(x, rp, rs, rt)
    check_linear(bf16_host(y)[:, cols], y_ref, bound, f"{wname} m={m}")


# ---------------------------------------------------------------------------
# Expert stacks (MoE layers) and the routed decode linear.
# ---------------------------------------------------------------------------
def _expert_stack(e, n, k, seed):
    """e experts with amaxes spread over a factor of ~5 (each expert gets its own tensor scale)."""
    return np.stack([WL.normal_bf16((n, k), 0.02 * (1.0 + 0.7 * i), seed + i) for i in range(e)])


@pytest.mark.parametrize("e,n,k", [(3, 48, 272), (4, 33, 5120), (1, 16, 16)])
def test_quantize_experts_bit_exact(nv, e, n, k):
    w = _expert_stack(e, n, k, 900 + k)
    packed, scales, tscale = nv.quantize_experts(to_dev_bf16(w))
    rp, rs, rt = O.quantize_experts(w)
    assert np.array_equal(tscale.cpu().numpy().view(np.uint32), rt.view(np.uint32))
    assert np.array_equal(u8_host(scales), rs)
    assert np.array_equal(u8_host(packed), rp)
    assert np.array_equal(bf16_host(nv.dequant_experts(packed, scales, tscale)), O.dequant_experts(rp, rs, rt))
    # matrix i equals the single-matrix quantizer on w[i]
    for i in range(e):
        qi = nv.quantize(to_dev_bf16(w[i]))
        assert torch.equal(qi[0], packed[i]) and torch.equal(qi[1], scales[i]) and torch.equal(qi[2][0], tscale[i])


# (tokens, topk, experts, n, k): K split GEMV (k = 5120, 2048, 512), and the loop GEMV
# (k = 1040: 8-byte units; k = 768: 16-byte units); ragged n.
ROUTED_SHAPES = [(1, 8, 16, 300, 5120), (3, 4, 6, 100, 2048), (2, 3, 5, 70, 1040), (4, 2, 3, 33, 768),
                 (5, 2, 4, 21, 512), (1, 1, 1, 16, 16)]


@pytest.mark.parametrize("t,topk,e,n,k", ROUTED_SHAPES)
def test_linear_routed(nv, t, topk, e, n, k):
    w = _expert_stack(e, n, k, 1000 + k)
    packed, scales, tscale = nv.quantize_experts(to_dev_bf16(w))
    rq = O.quantize_experts(w)
    assert np.array_equal(u8_host(packed), rq[0]) and np.array_equal(u8_host(scales), rq[1])
    x = WL.normal_bf16((t, k), 1.0, 1100 + t)
    rng = np.random.default_rng(1200 + e)
    route = rng.integers(0, e, size=(t, topk)).astype(np.int32)
    if t * topk >= 3:
        route.flat[1] = route.flat[0]   # the same expert twice
        route.flat[2] = -1              # out of range: zeros
    if t * topk >= 4:
        route.flat[3] = e               # out of range: zeros
    y = nv.linear_routed(to_dev_bf16(x), torch.from_numpy(route).cuda(), packed, scales, tscale)
    y_ref, bound = O.linear_routed_ref(x, route, *rq)
    yb = bf16_host(y)
    check_linear(yb.reshape(t * topk, n), y_ref.reshape(t * topk, n), bound.reshape(t * topk, n),
                 f"routed t={t} topk={topk} e={e} n={n} k={k}")
    bad = (route < 0) | (route >= e)
    assert np.all(yb[bad] == 0), "out-of-range expert ids must give zero rows"
    # deterministic; and, where the routed path runs the K-split GEMV, the same bits as the
    # plain GEMV on the chosen expert
    assert torch.equal(nv.linear_routed(to_dev_bf16(x), torch.from_numpy(route).cuda(), packed, scales, tscale), y)
    if k % 512 == 0 and k <= 5120:
        for (ti, j) in [(0, 0), (t - 1, topk - 1)]:
            ei = int(route[ti, j])
            if 0 <= ei < e:
                yg = nv.linear(to_dev_bf16(x[ti:ti + 1]), packed[ei], scales[ei], tscale[ei:ei + 1].clone(),
                               kernel="gemv")
                assert np.array_equal(bf16_host(yg)[0], yb[ti, j])


def test_linear_routed_edges(nv):
    w = _expert_stack(2, 16, 512, 1300)
    packed, scales, tscale = nv.quantize_experts(to_dev_bf16(w))
    # t = 0 is a no-op
    y = nv.linear_routed(torch.empty((0, 512), dtype=torch.bfloat16, device="cuda"),
                         torch.empty((0, 3), dtype=torch.int32, device="cuda"), packed, scales, tscale)
    assert y.shape == (0, 3, 16)
    # every id out of range: all zeros, nothing read from the stack
    x = to_dev_bf16(WL.normal_bf16((2, 512), 1.0, 1301))
    bad = torch.tensor([[-5, 2], [7, 2 ** 31 - 1]], dtype=torch.int32, device="cuda")
    assert torch.count_nonzero(nv.linear_routed(x, bad, packed, scales, tscale)) == 0
    # argument errors are reported before anything is launched
    from nvfp4_weight_only_amd import binding as B
    y = torch.empty((2, 2, 16), dtype=torch.bfloat16, device="cuda")
    args = lambda topk, e, yp: (x.data_ptr(), 2, topk, bad.data_ptr(), e, 16, 512, packed.data_ptr(),  # noqa: E731
                                scales.data_ptr(), tscale.data_ptr(), yp, 0)
    assert nv.lib().nvfp4_linear_routed(*args(0, 2, y.data_ptr())) == B.ERR_SHAPE
    assert nv.lib().nvfp4_linear_routed(*args(2, 0, y.data_ptr())) == B.ERR_SHAPE
    assert nv.lib().nvfp4_linear_routed(*args(2, 2, x.data_ptr())) == B.ERR_ALIAS   # y overlaps x
    assert nv.lib().nvfp4_linear_routed(*args(2, 2, y.data_ptr() + 2)) == B.ERR_ALIGN


# ---------------------------------------------------------------------------
# Grouped (prefill) form over an expert stack: pairs sorted by expert on the
# device, 128-row tiles per expert.  Same oracle as the routed decode.
# ---------------------------------------------------------------------------
def _routing(kind, t, topk, e, seed):
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        r = rng.integers(0, e, size=(t, topk))
    elif kind == "skew":        # geometric: expert 0 takes about half of the pairs, the last ones few or none
        r = np.minimum(rng.geometric(0.5, size=(t, topk)) - 1, e - 1)
    else:                       # "one": every pair on expert 1, the other experts empty
        r = np.ones((t, topk), dtype=np.int64)
    r = r.astype(np.int32)
    if t * topk >= 6:
        r.flat[2] = -1
        r.flat[3] = e
        r.flat[5] = 2 ** 31 - 1
    return r


GROUPED_CASES = [
    (300, 4, 6, 300, 1024, "uniform"),   # ~200 pairs per expert: 2 tiles each, the second ragged; n = 272 + 28
    (200, 8, 16, 545, 256, "skew"),      # one expert with 6+ tiles, experts with a few rows or none
    (130, 2, 3, 64, 512, "one"),         # 257 pairs on one expert (3 tiles, the last 1 row); 2 empty experts
    (1, 1, 1, 16, 256, "uniform"),       # one pair
    (40, 3, 5, 100, 1040, "uniform"),    # k % 256 != 0: the routed GEMV runs instead
    (4200, 8, 4, 16, 256, "uniform"),    # 33600 pairs: more than the sort keeps in LDS
]


@pytest.mark.parametrize("t,topk,e,n,k,kind", GROUPED_CASES)
def test_linear_grouped(nv, t, topk, e, n, k, kind):
    w = _expert_stack(e, n, k, 1400 + k)
    packed, scales, tscale = nv.quantize_experts(to_dev_bf16(w))
    rq = O.quantize_experts(w)
    assert np.array_equal(u8_host(packed), rq[0]) and np.array_equal(u8_host(scales), rq[1])
    x = WL.normal_bf16((t, k), 1.0, 1500 + t)
    route = _routing(kind, t, topk, e, 1600 + e)
    xd, rd = to_dev_bf16(x), torch.from_numpy(route).cuda()
    y = nv.linear_grouped(xd, rd, packed, scales, tscale)
    y_ref, bound = O.linear_routed_ref(x, route, *rq)
    yb = bf16_host(y)
    check_linear(yb.reshape(t * topk, n), y_ref.reshape(t * topk, n), bound.reshape(t * topk, n),
                 f"grouped t={t} topk={topk} e={e} n={n} k={k} {kind}")
    bad = (route < 0) | (route >= e)
    assert np.all(yb[bad] == 0), "out-of-range expert ids must give zero rows"
    # the sort order inside an expert varies between calls; the output does not
    assert torch.equal(nv.linear_grouped(xd, rd, packed, scales, tscale), y)
    if k % 256 == 0:
        # each row is the dense prefill GEMM's row for that token and expert, bit for bit
        for ei in np.unique(route[~bad])[:3]:
            ts, js = np.nonzero(route == ei)
            yd = nv.linear(to_dev_bf16(x[ts]), packed[ei], scales[ei], tscale[ei:ei + 1].clone(), kernel="prefill")
            assert np.array_equal(bf16_host(yd), yb[ts, js]), f"expert {ei}"
    else:
        assert torch.equal(nv.linear_routed(xd, rd, packed, scales, tscale), y)


def test_linear_grouped_workspace_reuse(nv):
    """One workspace, two calls in a row (the second with fewer tokens and other ids): the counters restart."""
    e, n, k = 4, 80, 512
    w = _expert_stack(e, n, k, 1700)
    packed, scales, tscale = nv.quantize_experts(to_dev_bf16(w))
    rq = O.quantize_experts(w)
    ws = torch.full((nv.linear_grouped_workspace_bytes(300, 3, e),), 0xAB, dtype=torch.uint8, device="cuda")
    for (t, topk, seed) in [(300, 3, 1701), (70, 2, 1702)]:
        x = WL.normal_bf16((t, k), 1.0, seed)
        route = _routing("uniform", t, topk, e, seed)
        y = nv.linear_grouped(to_dev_bf16(x), torch.from_numpy(route).cuda(), packed, scales, tscale, workspace=ws)
        y_ref, bound = O.linear_routed_ref(x, route, *rq)
        check_linear(bf16_host(y).reshape(t * topk, n), y_ref.reshape(t * topk, n), bound.reshape(t * topk, n),
                     f"grouped workspace reuse t={t} topk={topk}")


def test_linear_grouped_edges(nv):
    from nvfp4_weight_only_amd import binding as B
    w = _expert_stack(2, 16, 512, 1800)
    packed, scales, tscale = nv.quantize_experts(to_dev_bf16(w))
    # t = 0 is a no-op
    y = nv.linear_grouped(torch.empty((0, 512), dtype=torch.bfloat16, device="cuda"),
                          torch.empty((0, 3), dtype=torch.int32, device="cuda"), packed, scales, tscale)
    assert y.shape == (0, 3, 16)
    # every id out of range: all zeros (no tile is scheduled)
    x = to_dev_bf16(WL.normal_bf16((2, 512), 1.0, 1801))
    bad = torch.tensor([[-5, 2], [7, 2 ** 31 - 1]], dtype=torch.int32, device="cuda")
    y = torch.full((2, 2, 16), 1.0, dtype=torch.bfloat16, device="cuda")
    assert torch.count_nonzero(nv.linear_grouped(x, bad, packed, scales, tscale, out=y)) == 0
    # argument errors are reported before anything is launched
    ws = torch.empty(nv.linear_grouped_workspace_bytes(2, 2, 2), dtype=torch.uint8, device="cuda")
    args = lambda yp, wp, wb: (x.data_ptr(), 2, 2, bad.data_ptr(), 2, 16, 512, packed.data_ptr(),  # noqa: E731
                               scales.data_ptr(), tscale.data_ptr(), yp, wp, wb, 0)
    L = nv.lib()
    assert L.nvfp4_linear_grouped(*args(y.data_ptr(), None, ws.numel())) == B.ERR_NULL
    assert L.nvfp4_linear_grouped(*args(y.data_ptr(), ws.data_ptr(), ws.numel() - 16)) == B.ERR_SHAPE
    assert L.nvfp4_linear_grouped(*args(y.data_ptr(), ws.data_ptr() + 8, ws.numel())) == B.ERR_ALIGN
    assert L.nvfp4_linear_grouped(*args(y.data_ptr(), y.data_ptr(), ws.numel())) == B.ERR_ALIAS
    assert L.nvfp4_linear_grouped(*args(x.data_ptr(), ws.data_ptr(), ws.numel())) == B.ERR_ALIAS


def test_linear_grouped_full_size_sampled(nv):
    """2048 tokens routed top-8 over 128 experts of 2048 x 4096 (the grouped prefill workload, launched as
    timed): sampled (pair, column) outputs against the oracle on those weight rows."""
    mw = WL.MOE_PREFILL
    base_bits = mw.base_weight()
    base = to_dev_bf16(base_bits)
    stack = torch.stack([(base.float() * mw.expert_scale(i)).to(torch.bfloat16) for i in range(mw.experts)])
    del base
    packed, scales, tscale = nv.quantize_experts(stack)
    route = mw.random_routes()
    x = WL.activations(mw.t, mw.k)
    y = bf16_host(nv.linear_grouped(to_dev_bf16(x), torch.from_numpy(route).cuda(), packed, scales, tscale))
    rng = np.random.default_rng(1900)
    cols = np.sort(rng.choice(mw.n, 24, replace=False))
    for ei in [0, 77, 127]:
        wb = mw.expert_weight(ei, base_bits)
        assert np.array_equal(bf16_host(stack[ei]), wb), "device-built expert differs from its definition"
        amax = O.tensor_amax(wb)
        q = O.quantize(wb[cols], amax=amax)
        ts, js = np.nonzero(route == ei)
        y_ref, bound = O.linear_ref(x[ts], *q)
        check_linear(y[ts, js][:, cols], y_ref, bound, f"grouped full size, expert {ei} ({ts.size} pairs)")
    del stack


@pytest.mark.parametrize("e", [2000, 9000])
def test_linear_grouped_many_experts(nv, e):
    """2000 experts: LDS counters, permutation stored straight to the workspace; 9000: more than the
    sort's LDS counters hold, so its counters live in the workspace too."""
    n, k, t, topk = 32, 256, 64, 4
    rng = np.random.default_rng(2000)
    w = WL.bf16_bits_from_f32((rng.standard_normal((e, n, k)) * 0.02 * (1.0 + rng.random((e, 1, 1)))).astype(np.float32))
    packed, scales, tscale = nv.quantize_experts(to_dev_bf16(w))
    x = WL.normal_bf16((t, k), 1.0, 2001)
    route = rng.integers(0, e, size=(t, topk)).astype(np.int32)
    route[0, :] = 17                   # several pairs on one expert
    route.flat[5] = -3
    route.flat[6] = e
    y = bf16_host(nv.linear_grouped(to_dev_bf16(x), torch.from_numpy(route).cuda(), packed, scales, tscale))
    ph, sh, th = u8_host(packed), u8_host(scales), tscale.cpu().numpy()
    for ti in range(t):
        for j in range(topk):
            ei = int(route[ti, j])
            if not 0 <= ei < e:
                assert np.all(y[ti, j] == 0)
                continue
            q = O.quantize(w[ei])
            assert np.array_equal(ph[ei], q[0]) and np.array_equal(sh[ei], q[1]) and th[ei] == q[2]
            y_ref, bound = O.linear_ref(x[ti:ti + 1], *q)
            bad = O.linear_violations(WL.f32_from_bf16_bits(y[ti, j][None]).astype(np.float64), y_ref, bound)
            assert not bad.any(), f"pair ({ti}, {j}) on expert {ei}: {int(bad.sum())} outputs outside 2e-3*B"


# ---------------------------------------------------------------------------
# Paged FP4 KV-cache gather: bit-exact against the oracle (R14-R16).
# ---------------------------------------------------------------------------
from oracle import kv_oracle as KV  # noqa: E402

KV_OUT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _kv_random_cache(fmt, nb, bs, heads, hd, seed):
    g = KV.GROUP[fmt]
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(nb, bs, heads, hd // 2), dtype=np.uint8)
    if fmt == KV.NVFP4:
        scales = rng.integers(0, 0x7F, size=(nb, bs, heads, hd // g), dtype=np.uint8)   # every finite E4M3
    else:
        scales = rng.integers(100, 155, size=(nb, bs, heads, hd // g), dtype=np.uint8)
        scales.flat[:6] = [0, 1, 126, 127, 141, 254]    # subnormal products, FP16 overflow, FP32 overflow
    return codes, scales


def _kv_run(nv, fmt, out, codes, scales, ts, table, lens, dst, out_rows, init_bits):
    od = KV_OUT[out]
    y = torch.from_numpy(init_bits.view(np.int16)).cuda().view(od)
    tsd = torch.tensor([ts], dtype=torch.float32, device="cuda") if fmt == KV.NVFP4 else None
    nv.kv_gather(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), tsd,
                 torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), torch.from_numpy(dst).cuda(), y,
                 fmt=fmt)
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def _kv_equal(got, want, out):
    """Bit equality, except that any NaN matches any NaN (payloads are not specified)."""
    dt = np.float16 if out == "f16" else None
    if dt is not None:
        gn, wn = np.isnan(got.view(np.float16)), np.isnan(want.view(np.float16))
    else:
        f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)  # noqa: E731
        gn, wn = np.isnan(f(got)), np.isnan(f(want))
    return np.array_equal(gn, wn) and np.array_equal(got[~gn], want[~wn])


KV_CASES = [   # nb, bs, heads, hd, lens, max_blocks
    (40, 16, 8, 128, [1, 17, 100, 0, 250], 16),
    (13, 7, 3, 64, [20, 49, 5], 7),
    (9, 1, 1, 32, [3, 9, 1], 9),
]


@pytest.mark.parametrize("fmt", [KV.NVFP4, KV.MXFP4])
@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("case", range(len(KV_CASES)))
def test_kv_gather(nv, fmt, out, case):
    nb, bs, heads, hd, lens, mb = KV_CASES[case]
    codes, scales = _kv_random_cache(fmt, nb, bs, heads, hd, 2100 + case)
    rng = np.random.default_rng(2200 + case)
    seqs = len(lens)
    table = rng.integers(0, nb, size=(seqs, mb)).astype(np.int32)      # pages shared and reused across sequences
    lens = np.array(lens, dtype=np.int32)
    dst = np.concatenate([[3], 3 + np.cumsum(lens + 5)[:-1]]).astype(np.int32)   # gaps for the current chunks
    out_rows = int(dst[-1] + lens[-1] + 4)
    init = rng.integers(0, 2 ** 16, size=(out_rows, heads, hd), dtype=np.uint16)
    ts = np.float32(0.0123)
    got = _kv_run(nv, fmt, out, codes, scales, ts, table, lens, dst, out_rows, init)
    want = KV.kv_gather_ref(fmt, out, codes, scales, ts, table, lens, dst, init)
    assert _kv_equal(got, want, out), f"{fmt} {out} case {case}: {int((got != want).sum())} elements differ"


@pytest.mark.parametrize("fmt", [KV.NVFP4, KV.MXFP4])
def test_kv_gather_edges(nv, fmt):
    """Out-of-range page ids (zeros), negative and over-long lengths, rows before 0 and past the end, NaN scale
    bytes; seqs = 0 is a no-op."""
    nb, bs, heads, hd = 6, 4, 2, 64
    codes, scales = _kv_random_cache(fmt, nb, bs, heads, hd, 2300)
    scales[2, 1, 0, 0] = 0x7F if fmt == KV.NVFP4 else 0xFF          # a NaN scale
    table = np.array([[3, -1, 2], [9, 2, 0], [2, 2, 2], [1, 0, 5], [4, 4, 4]], dtype=np.int32)
    lens = np.array([12, 9, -4, 40, 7], dtype=np.int32)
    dst = np.array([-3, 10, 30, 22, 38], dtype=np.int32)
    out_rows = 42
    for out in ("f16", "bf16"):
        init = np.full((out_rows, heads, hd), 0x3C00 if out == "f16" else 0x3F80, dtype=np.uint16)
        got = _kv_run(nv, fmt, out, codes, scales, np.float32(0.5), table, lens, dst, out_rows, init)
        want = KV.kv_gather_ref(fmt, out, codes, scales, np.float32(0.5), table, lens, dst, init)
        assert _kv_equal(got, want, out), out
    y = torch.zeros((4, heads, hd), dtype=torch.float16, device="cuda")
    e = torch.empty((0, 3), dtype=torch.int32, device="cuda")
    nv.kv_gather(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                 torch.ones(1, device="cuda") if fmt == KV.NVFP4 else None, e,
                 torch.empty(0, dtype=torch.int32, device="cuda"), torch.empty(0, dtype=torch.int32, device="cuda"),
                 y, fmt=fmt)
    assert torch.count_nonzero(y) == 0


@pytest.mark.parametrize("fmt", [KV.NVFP4, KV.MXFP4])
def test_kv_gather_full_size_sampled(nv, fmt):
    """The chunked-prefill gather workload (16 sequences, 66,971 past tokens, 8 x 128, 16-token pages), launched
    as timed; three whole sequences (short, long, last) against the oracle."""
    kw = WL.KV_PREFILL
    table, lens, dst, nb, out_rows = kw.layout()
    codes, scales = kw.cache(fmt, nb)
    init = np.zeros((out_rows, kw.heads, kw.head_dim), dtype=np.uint16)
    got = _kv_run(nv, fmt, "f16", codes, scales, np.float32(kw.KV_TSCALE), table, lens, dst, out_rows, init)
    for s in (int(np.argmin(lens)), int(np.argmax(lens)), kw.seqs - 1):
        sel = slice(s, s + 1)
        want = KV.kv_gather_ref(fmt, "f16", codes, scales, np.float32(kw.KV_TSCALE), table[sel], lens[sel], dst[sel],
                                init)
        rows = slice(int(dst[s]), int(dst[s] + lens[s]))
        assert np.array_equal(got[rows], want[rows]), f"sequence {s}"
        assert not np.any(got[int(dst[s] + lens[s]):int(dst[s] + lens[s]) + kw.chunk]), "chunk rows must stay zero"


# ---------------------------------------------------------------------------
# MXFP4 tensors and the W4A4 GEMM (R17-R19).
# ---------------------------------------------------------------------------
from oracle import mxfp4_oracle as MXO  # noqa: E402


def _mx_inputs(rows, k, seed, spread=16):
    """BF16 rows whose 32-element blocks span 2^-spread .. 2^spread, with zero, negative-zero and subnormal
    blocks and exact midpoints mixed in."""
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((rows, k)).astype(np.float32)
    f *= np.exp2(rng.integers(-spread, spread + 1, size=(rows, k // 32, 1))).repeat(32, axis=2).reshape(rows, k)
    w = WL.bf16_bits_from_f32(f)
    if rows >= 3 and k >= 64:
        w[0, :32] = 0
        w[1, 32:64] = 0x8000
        w[2, :32] = WL.bf16_bits_from_f32((rng.random(32) * 2.0 ** -126).astype(np.float32))   # subnormal block
        w[2, 32:44] = WL.bf16_bits_from_f32(np.array([4, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, 6.5, 7.9, -5, -.75],
                                                     dtype=np.float32))
    return w


def _mx_dev(p, s):
    return torch.from_numpy(np.ascontiguousarray(p)).cuda(), torch.from_numpy(np.ascontiguousarray(s)).cuda()


@pytest.mark.parametrize("rows,k", [(64, 512), (37, 96), (1, 32), (300, 5120)])
def test_mx_quantize_bit_exact(nv, rows, k):
    w = _mx_inputs(rows, k, 3000 + k)
    packed, scales = nv.mx_quantize(to_dev_bf16(w))
    rp, rs = MXO.quantize(w)
    assert np.array_equal(u8_host(scales), rs)
    assert np.array_equal(u8_host(packed), rp)


def test_mx_dequant_bit_exact(nv):
    rng = np.random.default_rng(3100)
    packed = rng.integers(0, 256, size=(40, 64), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(40, 4), dtype=np.uint8)
    scales.flat[:5] = [0, 1, 127, 254, 255]
    got = bf16_host(nv.mx_dequant(*_mx_dev(packed, scales)))
    with np.errstate(over="ignore"):   # scale byte 254 times 6 overflows FP32 to inf, as the format says
        want = O.f32_to_bf16_rne(MXO.dequant_exact(packed, scales).astype(np.float32))
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    assert np.array_equal(np.isnan(f(got)), np.isnan(f(want)))
    ok = ~np.isnan(f(want))
    assert np.array_equal(got[ok], want[ok])


# 192-row weight tiles for most shapes; (16, 65536, 128) takes the 256-row tiles (one round of 256 of them
# against two rounds of 192-row tiles).
MX_GEMM_SHAPES = [(1, 16, 256), (33, 300, 512), (256, 256, 256), (300, 520, 1024), (513, 257, 768), (40, 64, 5120),
                  (48, 200, 384), (7, 33, 128), (16, 65536, 128)]


@pytest.mark.parametrize("m,n,k", MX_GEMM_SHAPES)
def test_mx_gemm(nv, m, n, k):
    """FP4 x FP4 GEMM on operands the oracle quantized, against the exact product of their values."""
    xp, xs = MXO.quantize(_mx_inputs(m, k, 3200 + m, spread=6))
    wp, wsc = MXO.quantize(_mx_inputs(n, k, 3300 + n, spread=6))
    y = bf16_host(nv.mx_gemm(*_mx_dev(xp, xs), *_mx_dev(wp, wsc)))
    xq, wq = MXO.dequant_exact(xp, xs), MXO.dequant_exact(wp, wsc)
    check_linear(y, xq @ wq.T, np.abs(xq) @ np.abs(wq).T, f"mx gemm {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(70, 300, 512), (2, 33, 256)])
def test_mx_linear_w4a4(nv, m, n, k):
    """BF16 X quantized on the GPU into the workspace (bit-exact against the oracle), then the GEMM."""
    x = _mx_inputs(m, k, 3400 + m, spread=4)
    wp, wsc = MXO.quantize(_mx_inputs(n, k, 3500 + n, spread=4))
    ws = torch.zeros(nv.lib().nvfp4_mx_linear_w4a4_workspace_bytes(m, k), dtype=torch.uint8, device="cuda")
    y = bf16_host(nv.mx_linear_w4a4(to_dev_bf16(x), *_mx_dev(wp, wsc), workspace=ws))
    rp, rs = MXO.quantize(x)
    wsh = u8_host(ws)
    pb = (m * k // 2 + 15) // 16 * 16
    assert np.array_equal(wsh[:m * k // 2].reshape(m, k // 2), rp)
    assert np.array_equal(wsh[pb:pb + m * k // 32].reshape(m, k // 32), rs)
    y_ref, bound = MXO.linear_w4a4_ref(x, wp, wsc)
    check_linear(y, y_ref, bound, f"mx w4a4 {m}x{n}x{k}")


def test_mx_gemm_edges(nv):
    from nvfp4_weight_only_amd import binding as B
    xp, xs = _mx_dev(*MXO.quantize(_mx_inputs(4, 320, 3600)))
    wp, wsc = _mx_dev(*MXO.quantize(_mx_inputs(8, 320, 3601)))
    y = torch.empty((4, 8), dtype=torch.bfloat16, device="cuda")
    assert nv.lib().nvfp4_mx_gemm(xp.data_ptr(), xs.data_ptr(), 4, wp.data_ptr(), wsc.data_ptr(), 8, 320,
                                  y.data_ptr(), 0) == B.ERR_UNSUPPORTED          # k % 256 != 0
    assert nv.lib().nvfp4_mx_gemm(xp.data_ptr(), xs.data_ptr(), 0, wp.data_ptr(), wsc.data_ptr(), 8, 320,
                                  y.data_ptr(), 0) == B.OK                       # m = 0


def test_mx_gemm_full_size_sampled(nv):
    """The W4A4 prefill workload (M=2048, N=17408, K=5120), launched as timed; sampled rows and columns
    against the oracle (MXFP4 blocks run along K, so a row's quantization does not depend on other rows)."""
    wl = WL.WORKLOADS["prefill"]
    m, n, k = 2048, wl.n, wl.k
    w = wl.weight()
    x = wl.activations(m)
    wq, wsc = nv.mx_quantize(to_dev_bf16(w))
    y = bf16_host(nv.mx_linear_w4a4(to_dev_bf16(x), wq, wsc))
    rng = np.random.default_rng(3700)
    rows = np.sort(rng.choice(m, 24, replace=False))
    cols = np.sort(np.concatenate([rng.choice(n, 40, replace=False), [0, n - 1]]))
    wp_s, ws_s = MXO.quantize(w[cols])
    assert np.array_equal(u8_host(wq)[cols], wp_s) and np.array_equal(u8_host(wsc)[cols], ws_s)
    y_ref, bound = MXO.linear_w4a4_ref(x[rows], wp_s, ws_s)
    check_linear(y[np.ix_(rows, cols)], y_ref, bound, "mx w4a4 full size, sampled")


# ---------------------------------------------------------------------------
# NVFP4 x NVFP4 linear: X quantized to NVFP4 on the stream, product on the
# BF16 matrix cores from X's exact E2M1 * E4M3 values.
# ---------------------------------------------------------------------------
def _w4a4_workspace_check(ws, x, m, k, tscale_w=None):
    """The workspace's X codes, scales, tensor amax / scale and decoded values against the oracle."""
    rp, rs, rt = O.quantize(x)
    h = u8_host(ws)
    r16 = lambda b: (b + 15) // 16 * 16
    o_s = r16(m * k // 2)
    o_f = o_s + r16(m * k // 16)
    assert np.array_equal(h[:m * k // 2].reshape(m, k // 2), rp), "X codes differ"
    assert np.array_equal(h[o_s:o_s + m * k // 16].reshape(m, k // 16), rs), "X scales differ"
    f = h[o_f:o_f + 16].view(np.float32)
    assert f[1] == np.float32(O.tensor_amax(x)), "X amax differs"
    assert f[2].view(np.uint32) == np.float32(rt).view(np.uint32), "X tensor scale differs"
    if tscale_w is not None:   # the output scale fl32(ts_w * ts_x)
        assert f[0].view(np.uint32) == (np.float32(tscale_w) * np.float32(rt)).view(np.uint32)
    dec = h[o_f + 16:o_f + 16 + 2 * m * k].view(np.uint16).reshape(m, k)
    want = O.f32_to_bf16_rne(O.decoded_products(rp, rs).astype(np.float32))   # exact: <= 6 significant bits
    assert np.array_equal(dec, want), f"{int((dec != want).sum())} decoded X values differ"


W4A4_SHAPES = [(1, 256, 512), (3, 300, 1040), (8, 272, 1024), (17, 130, 272), (33, 200, 512), (300, 272, 1024),
               (130, 64, 5120)]


@pytest.mark.parametrize("m,n,k", W4A4_SHAPES)
def test_linear_w4a4(nv, m, n, k):
    x = WL.normal_bf16((m, k), 1.0, 3800 + m)
    w = WL.normal_bf16((n, k), 0.02, 3900 + n)
    (packed, scales, tscale), (rp, rs, rt) = q_both(nv, w)
    ws = torch.empty(nv.linear_w4a4_workspace_bytes(m, k), dtype=torch.uint8, device="cuda")
    y = bf16_host(nv.linear_w4a4(to_dev_bf16(x), packed, scales, tscale, workspace=ws))
    _w4a4_workspace_check(ws, x, m, k, rt)
    y_ref, bound = O.linear_w4a4_ref(x, rp, rs, rt)
    check_linear(y, y_ref, bound, f"nvfp4 w4a4 {m}x{n}x{k}")
    y2 = bf16_host(nv.linear_w4a4(to_dev_bf16(x), packed, scales, tscale, workspace=ws))
    assert np.array_equal(y, y2), "not deterministic"


def test_linear_w4a4_edges(nv):
    w = WL.normal_bf16((64, 512), 0.02, 3950)
    (packed, scales, tscale), _ = q_both(nv, w)
    # all-zero X: tensor scale 0, every code and value 0, Y = 0
    x0 = np.zeros((5, 512), dtype=np.uint16)
    ws = torch.empty(nv.linear_w4a4_workspace_bytes(5, 512), dtype=torch.uint8, device="cuda").fill_(0xAB)
    y = bf16_host(nv.linear_w4a4(to_dev_bf16(x0), packed, scales, tscale, workspace=ws))
    assert not y.any()
    _w4a4_workspace_check(ws, x0, 5, 512)
    # m = 0 is a no-op
    e = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    assert nv.linear_w4a4(e, packed, scales, tscale).shape == (0, 64)
    # one huge outlier: the rest of X rounds to small codes or zero, still within the bound of X_hat
    x = WL.normal_bf16((4, 512), 1.0, 3951)
    x[2, 100] = WL.bf16_bits_from_f32(np.array([3.0e4], dtype=np.float32))[0]
    y = bf16_host(nv.linear_w4a4(to_dev_bf16(x), packed, scales, tscale))
    y_ref, bound = O.linear_w4a4_ref(x, *O.quantize(w))
    check_linear(y, y_ref, bound, "nvfp4 w4a4 outlier")


def test_linear_w4a4_full_size_sampled(nv):
    """The prefill workload (M=2048, N=17408, K=5120) with NVFP4 activations, launched as timed; sampled rows
    and columns against the oracle, which quantizes the sampled rows against the whole X's amax."""
    wl = WL.WORKLOADS["prefill"]
    m, n, k = 2048, wl.n, wl.k
    (packed, scales, tscale), w, amax = _quantized(nv, "prefill")
    x = wl.activations(m)
    y = bf16_host(nv.linear_w4a4(to_dev_bf16(x), packed, scales, tscale))
    rng = np.random.default_rng(3960)
    rows = np.sort(np.concatenate([rng.choice(m, 24, replace=False), [0, m - 1]]))
    cols = sample_rows(n, 40, seed=3961)
    rp, rs, rt = O.quantize(w[cols], amax=amax)
    assert np.array_equal(u8_host(packed)[cols], rp) and np.array_equal(u8_host(scales)[cols], rs)
    y_ref, bound = O.linear_w4a4_ref(x[rows], rp, rs, rt, x_amax=O.tensor_amax(x))
    check_linear(y[np.ix_(rows, cols)], y_ref, bound, "nvfp4 w4a4 full size, sampled")


# ---------------------------------------------------------------------------
# HIP-graph capture: every entry point captured once and replayed several
# times, with eager work and synchronizations between the replays; each
# replay must give the eager result bit for bit.
# ---------------------------------------------------------------------------
def test_graph_replays_match_eager(nv):
    torch.manual_seed(0)
    st = torch.cuda.Stream()
    wd = to_dev_bf16(WL.normal_bf16((272, 1024), 0.02, 4000))
    with torch.cuda.stream(st):
        p, s, t = nv.quantize(wd)
    torch.cuda.synchronize()
    x1 = to_dev_bf16(WL.normal_bf16((1, 1024), 1.0, 4001))
    x8 = to_dev_bf16(WL.normal_bf16((8, 1024), 1.0, 4002))
    x300 = to_dev_bf16(WL.normal_bf16((300, 1024), 1.0, 4003))
    stack = to_dev_bf16(_expert_stack(4, 80, 512, 4004))
    route = torch.from_numpy(_routing("uniform", 150, 3, 4, 4005)).cuda()
    xg = to_dev_bf16(WL.normal_bf16((150, 512), 1.0, 4006))
    gws = torch.empty(nv.linear_grouped_workspace_bytes(150, 3, 4), dtype=torch.uint8, device="cuda")
    codes, kscales = _kv_random_cache(KV.NVFP4, 12, 16, 2, 64, 4007)
    kc, ks_ = torch.from_numpy(codes).cuda(), torch.from_numpy(kscales).cuda()
    table = torch.from_numpy(np.random.default_rng(4008).integers(0, 12, size=(3, 4)).astype(np.int32)).cuda()
    klen = torch.tensor([20, 64, 5], dtype=torch.int32, device="cuda")
    kdst = torch.tensor([0, 24, 90], dtype=torch.int32, device="cuda")
    kts = torch.tensor([0.25], dtype=torch.float32, device="cuda")
    mxw = nv.mx_quantize(to_dev_bf16(_mx_inputs(256, 512, 4009, spread=4)))
    xm = to_dev_bf16(_mx_inputs(64, 512, 4010, spread=4))
    mws = torch.empty(nv.lib().nvfp4_mx_linear_w4a4_workspace_bytes(64, 512), dtype=torch.uint8, device="cuda")
    ep, es, et = nv.quantize_experts(stack)
    w64 = to_dev_bf16(WL.normal_bf16((64, 5120), 0.02, 4011))
    p64, s64, t64 = nv.quantize(w64)
    x24 = to_dev_bf16(WL.normal_bf16((24, 5120), 1.0, 4012))
    torch.cuda.synchronize()

    outs = {
        "gemv": torch.empty((1, 272), dtype=torch.bfloat16, device="cuda"),
        "small_m": torch.empty((8, 272), dtype=torch.bfloat16, device="cuda"),
        "prefill": torch.empty((300, 272), dtype=torch.bfloat16, device="cuda"),
        "dequant": torch.empty((272, 1024), dtype=torch.bfloat16, device="cuda"),
        "routed": torch.empty((150, 3, 80), dtype=torch.bfloat16, device="cuda"),
        "grouped": torch.empty((150, 3, 80), dtype=torch.bfloat16, device="cuda"),
        "kv": torch.empty((100, 2, 64), dtype=torch.float16, device="cuda"),
        "w4a4": torch.empty((64, 256), dtype=torch.bfloat16, device="cuda"),
        "nv_w4a4": torch.empty((300, 272), dtype=torch.bfloat16, device="cuda"),
        # kernel-native layout: the conversion, its dequantizer, the GEMV, the small-M kernel and its
        # activations-through-LDS form with a K split (64 x 5120 at m = 24: five slices)
        "prep": torch.empty(nv.lib().nvfp4_prepared_bytes(272, 1024), dtype=torch.uint8, device="cuda"),
        "prep64": torch.empty(nv.lib().nvfp4_prepared_bytes(64, 5120), dtype=torch.uint8, device="cuda"),
        "dq_prep": torch.empty((272, 1024), dtype=torch.bfloat16, device="cuda"),
        "prep_gemv": torch.empty((1, 272), dtype=torch.bfloat16, device="cuda"),
        "prep_small_m": torch.empty((8, 272), dtype=torch.bfloat16, device="cuda"),
        "prep_xl_split": torch.empty((24, 64), dtype=torch.bfloat16, device="cuda"),
    }
    nws = torch.empty(nv.linear_w4a4_workspace_bytes(300, 1024), dtype=torch.uint8, device="cuda")
    quant = {}

    def step():
        L = nv.lib()
        sid = st.cuda_stream
        nv.linear(x1, p, s, t, out=outs["gemv"])
        nv.linear(x8, p, s, t, out=outs["small_m"])
        nv.linear(x300, p, s, t, out=outs["prefill"])
        assert L.nvfp4_dequant(p.data_ptr(), s.data_ptr(), t.data_ptr(), 272, 1024, outs["dequant"].data_ptr(),
                               sid) == 0
        if "p" not in quant:
            quant["p"] = torch.empty_like(p)
            quant["s"] = torch.empty_like(s)
            quant["t"] = torch.empty_like(t)
        assert L.nvfp4_quantize(wd.data_ptr(), 272, 1024, quant["p"].data_ptr(), quant["s"].data_ptr(),
                                quant["t"].data_ptr(), sid) == 0
        nv.linear_routed(xg, route, ep, es, et, out=outs["routed"])
        nv.linear_grouped(xg, route, ep, es, et, out=outs["grouped"], workspace=gws)
        nv.kv_gather(kc, ks_, kts, table, klen, kdst, outs["kv"], fmt="nvfp4")
        nv.mx_linear_w4a4(xm, mxw[0], mxw[1], out=outs["w4a4"], workspace=mws)
        nv.linear_w4a4(x300, p, s, t, out=outs["nv_w4a4"], workspace=nws)
        assert L.nvfp4_prepare(p.data_ptr(), s.data_ptr(), 272, 1024, outs["prep"].data_ptr(), sid) == 0
        assert L.nvfp4_prepare(p64.data_ptr(), s64.data_ptr(), 64, 5120, outs["prep64"].data_ptr(), sid) == 0
        assert L.nvfp4_dequant_prepared(outs["prep"].data_ptr(), t.data_ptr(), 272, 1024, outs["dq_prep"].data_ptr(),
                                        sid) == 0
        nv.linear_prepared(x1, outs["prep"], t, 272, out=outs["prep_gemv"])
        nv.linear_prepared(x8, outs["prep"], t, 272, out=outs["prep_small_m"])
        nv.linear_prepared(x24, outs["prep64"], t64, 64, out=outs["prep_xl_split"])

    with torch.cuda.stream(st):
        for o in outs.values():
            o.zero_()
        step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    eager.update({"q_" + k: v.clone() for k, v in quant.items()})
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in list(outs.values()) + list(quant.values()):
            o.zero_()                                     # eager work between replays
        nv.linear(x8, p, s, t)                            # an eager call on the default stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.int16), eager[k].view(torch.int16)), f"replay {rep}: {k}"
        for k, v in quant.items():
            assert torch.equal(v, eager["q_" + k]), f"replay {rep}: quantize {k}"


def test_graph_keeps_binding_workspace_after_growth(nv):
    """A graph captured with the binding's split-K workspace stays correct after a larger shape on the same
    stream grows that workspace: the old one is kept, so a tensor allocated afterwards cannot take its memory."""
    st = torch.cuda.Stream()
    m, n, k = 8, 300, 2048
    q, rq = q_both(nv, WL.normal_bf16((n, k), 0.02, 4100))
    x = WL.normal_bf16((m, k), 1.0, 4101)
    xd = to_dev_bf16(x)
    y_ref, bound = O.linear_ref(x, *rq)
    assert nv.linear_workspace_bytes(m, n, k) > 0, "shape expected to split K"
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(st):
        nv.linear(xd, *q, out=out)                       # allocates the stream's workspace eagerly
    torch.cuda.synchronize()
    eager = out.clone()
    check_linear(bf16_host(eager), y_ref, bound, "split-K before capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            nv.linear(xd, *q, out=out)
    torch.cuda.synchronize()
    # A larger split shape on the same stream grows the binding's workspace.
    m2, n2, k2 = 32, 5120, 4096
    big = nv.linear_workspace_bytes(m2, n2, k2)
    assert big > nv.linear_workspace_bytes(m, n, k)
    q2, _ = q_both(nv, WL.normal_bf16((n2, k2), 0.02, 4102))
    x2 = to_dev_bf16(WL.normal_bf16((m2, k2), 1.0, 4103))
    with torch.cuda.stream(st):
        nv.linear(x2, *q2)
    torch.cuda.synchronize()
    sentinel = torch.full((1 << 20,), 0x5A, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert bool((sentinel == 0x5A).all()), f"replay {rep} wrote into a later allocation"


# ---------------------------------------------------------------------------
# Prefill tile counts a little past whole rounds of 256 (q rounds and r <= 128
# more: 256 q whole tiles, then the rest split along K, launched after them):
# the whole output against the oracle, the same bits on a second call, and the
# unsplit call (no workspace) within the same tolerance.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n,k", [(4000, 2200, 512), (2049, 5120, 1024), (3500, 5120, 2048)])
def test_prefill_whole_then_split_tiles(nv, m, n, k):
    w = WL.normal_bf16((n, k), 0.02, 7900 + n)
    x = WL.normal_bf16((m, k), 1.0, 7950 + m)
    (packed, scales, tscale), rq = q_both(nv, w)
    y_ref, bound = O.linear_ref(x, *rq)
    xd = to_dev_bf16(x)
    need = nv.lib().nvfp4_linear_workspace_bytes(m, n, k)
    assert need > 0, "this shape takes the split"
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y1 = bf16_host(nv.linear(xd, packed, scales, tscale, workspace=ws))
    check_linear(y1, y_ref, bound, f"prefill split m={m} n={n} k={k}")
    assert np.array_equal(bf16_host(nv.linear(xd, packed, scales, tscale, workspace=ws)), y1)
    y0 = bf16_host(nv.linear(xd, packed, scales, tscale, workspace=None))
    check_linear(y0, y_ref, bound, f"prefill unsplit m={m} n={n} k={k}")


# ---------------------------------------------------------------------------
# Kernel-native layout (nvfp4_prepare): conversion bit-exact against the layout
# oracle, dequant bit-exact against the weight oracle, and the small-M linear
# on the prepared weight within the linear's tolerance.
# ---------------------------------------------------------------------------
from oracle import layout_oracle as LO  # noqa: E402

PREP_SHAPES = [(16, 128), (37, 384), (300, 1024), (5, 640), (64, 5120)]


@pytest.mark.parametrize("n,k", PREP_SHAPES)
def test_prepare_and_dequant_prepared_bit_exact(nv, n, k):
    w = WL.normal_bf16((n, k), 0.02, 7200 + n)
    (packed, scales, tscale), (rp, rs, rt) = q_both(nv, w)
    prep = nv.prepare(packed, scales)
    assert prep.numel() == LO.prepared_bytes(n, k)
    assert np.array_equal(u8_host(prep), LO.prepare(rp, rs)), "prepared layout differs from the oracle"
    dq = bf16_host(nv.dequant_prepared(prep, tscale, n, k))
    assert np.array_equal(dq, O.dequant(rp, rs, rt)), "dequant of the prepared layout differs from the oracle"


PREP_LINEAR = [(1, 16, 128), (2, 100, 128), (8, 300, 1024), (16, 37, 384), (17, 64, 5120), (32, 300, 640),
               (5, 1000, 384), (8, 10240, 512), (3, 2000, 8192), (32, 68, 1280), (24, 700, 3072),
               # m > 16 through LDS with 2 and 1 K slices, the last tile ragged; and m > 16 with more than 256
               # workgroups (two per CU), which keeps the activations in registers
               (20, 9000, 4096), (32, 17000, 2048), (24, 21000, 256),
               # m = 1 (the GEMV): fewer quads than wavefronts, 1 / 2 / 4 quads per chunk, two and three chunks,
               # an odd tile count under two tiles per workgroup, and the one-tile shape for many tiles
               (1, 37, 384), (1, 300, 2176), (1, 1000, 8192), (1, 33, 10240), (1, 70, 17408), (1, 16390, 512)]


@pytest.mark.parametrize("m,n,k", PREP_LINEAR)
def test_linear_prepared(nv, m, n, k):
    w = WL.normal_bf16((n, k), 0.02, 7300 + n)
    x = WL.normal_bf16((m, k), 1.0, 7400 + m)
    (packed, scales, tscale), rq = q_both(nv, w)
    prep = nv.prepare(packed, scales)
    y_ref, bound = O.linear_ref(x, *rq)
    xd = to_dev_bf16(x)
    y0 = bf16_host(nv.linear_prepared(xd, prep, tscale, n, workspace=None))
    check_linear(y0, y_ref, bound, f"prepared unsplit m={m} n={n} k={k}")
    need = nv.lib().nvfp4_linear_prepared_workspace_bytes(m, n, k)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    y1 = bf16_host(nv.linear_prepared(xd, prep, tscale, n, workspace=ws))
    check_linear(y1, y_ref, bound, f"prepared split m={m} n={n} k={k} (workspace {need} B)")
    for _ in range(2):   # counters back at zero; bitwise reproducible
        assert np.array_equal(bf16_host(nv.linear_prepared(xd, prep, tscale, n, workspace=ws)), y1)
        assert np.array_equal(bf16_host(nv.linear_prepared(xd, prep, tscale, n, workspace=None)), y0)


def test_linear_prepared_rejects_prefill_m(nv):
    w = WL.normal_bf16((32, 256), 0.02, 7500)
    packed, scales, tscale = nv.quantize(to_dev_bf16(w))
    prep = nv.prepare(packed, scales)
    with pytest.raises(nv.NVFP4Error):
        nv.linear_prepared(to_dev_bf16(WL.normal_bf16((33, 256), 1.0, 7501)), prep, tscale, 32)


PREP_FULL = [("small_m_up", 8), ("small_m_up", 32), ("small_m_down", 8), ("small_m_down", 32), ("gate_up", 1),
             ("decode", 1)]


@pytest.mark.parametrize("wname,m", PREP_FULL, ids=[f"{a}-m{b}" for a, b in PREP_FULL])
def test_linear_prepared_full_size_sampled(nv, wname, m):
    """The timed workloads on the prepared weight, launched as the benchmark does (binding workspace):
    sampled output columns against the oracle, and the prepared bytes of sampled tiles against the layout
    oracle."""
    wl = WL.WORKLOADS[wname]
    w = wl.weight()
    x = wl.activations(m)
    packed, scales, tscale = nv.quantize(to_dev_bf16(w))
    prep = nv.prepare(packed, scales)
    y = bf16_host(nv.linear_prepared(to_dev_bf16(x), prep, tscale, wl.n))
    amax = O.tensor_amax(w)
    tiles = np.unique(np.concatenate([sample_rows(wl.n // 16, 6, seed=7600), [0, wl.n // 16 - 1]]))
    rows = np.concatenate([np.arange(16 * t, 16 * t + 16) for t in tiles])
    rp, rs, rt = O.quantize(w[rows], amax=amax)
    ph = u8_host(prep).reshape(wl.k // 128, wl.n // 16, 1152)      # quad-major: [quad, tile, block]
    for j, t in enumerate(tiles):
        want = LO.prepare(rp[16 * j:16 * j + 16], rs[16 * j:16 * j + 16])   # one tile: its quads in order
        assert np.array_equal(ph[:, t, :].reshape(-1), want), f"tile {t}"
    y_ref, bound = O.linear_ref(x, rp, rs, rt)
    check_linear(y[:, rows], y_ref, bound, f"{wname} prepared m={m} full size, sampled")


def test_stream_read_reads_every_byte(nv):
    """The streaming-read measurement kernel folds every byte: the XOR of its per-workgroup sink words is the
    XOR of the whole buffer (computed on the host), at sizes with a ragged last workgroup and with more data
    than the grid covers in one pass."""
    rng = np.random.default_rng(7700)
    L = nv.lib()
    for nbytes in (16, 4096, 16 * 2049 * 256 + 48, 16 * 8192 * 2048 + 16 * 300):
        data = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
        want = int(np.bitwise_xor.reduce(data))
        src = torch.from_numpy(data.view(np.int32)).cuda()
        words = L.nvfp4_stream_read_sink_words(nbytes)
        assert 1 <= words <= 8192
        sink = torch.zeros(words + 4, dtype=torch.int32, device="cuda")
        assert L.nvfp4_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32)
        assert int(np.bitwise_xor.reduce(got[:words])) == want, nbytes
        assert not got[words:].any(), "wrote past its sink words"
