"""Host-side checks of libnvfp4.so: it loads, exports every declared symbol, and
validates arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

from nvfp4_weight_only_amd import binding as B
from nvfp4_weight_only_amd import build as BUILD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.lib_path()):
        BUILD.build()
    return B.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", B.lib_path()], check=True, capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_status_strings(L):
    for code in range(7):
        s = L.nvfp4_status_string(code).decode()
        assert s.startswith("NVFP4_")
    assert L.nvfp4_status_string(99).decode() == "NVFP4_ERR_UNKNOWN"
    assert L.nvfp4_version().decode().startswith("nvfp4-mi355x")


# Fake, never-dereferenced device addresses: validation fails before any HIP call.
A = 0x10000000
Bp = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000


def test_linear_validation(L):
    lin = L.nvfp4_linear
    assert lin(None, 1, 64, 64, Bp, C, D, E, None) == B.ERR_NULL
    assert lin(A, 1, 64, 24, Bp, C, D, E, None) == B.ERR_SHAPE          # k % 16 != 0
    assert lin(A, 1, 0, 64, Bp, C, D, E, None) == B.ERR_SHAPE           # n <= 0
    assert lin(A, -1, 64, 64, Bp, C, D, E, None) == B.ERR_SHAPE         # m < 0
    assert lin(A, 1, 64, 2 ** 62, Bp, C, D, E, None) == B.ERR_SHAPE     # size overflow
    assert lin(A + 8, 1, 64, 64, Bp, C, D, E, None) == B.ERR_ALIGN
    assert lin(A, 1, 64, 64, Bp, C, D + 4, E, None) == B.ERR_ALIGN
    assert lin(A, 4, 64, 64, Bp, C, D, A + 16, None) == B.ERR_ALIAS     # y overlaps x
    assert lin(A, 4, 64, 64, Bp, C, D, C, None) == B.ERR_ALIAS          # y overlaps scales
    assert lin(A, 0, 64, 64, Bp, C, D, E, None) == B.OK                 # m = 0 is a no-op
    assert lin(None, 0, 64, 64, Bp, C, D, None, None) == B.OK           # ... even with empty x and y
    assert lin(None, 0, 64, 64, None, C, D, None, None) == B.ERR_NULL
    assert lin(None, 0, 64, 24, Bp, C, D, None, None) == B.ERR_SHAPE
    assert L.nvfp4_linear_forced(7, A, 1, 64, 64, Bp, C, D, E, None) == B.ERR_UNSUPPORTED
    assert L.nvfp4_linear_forced(2, A, 1, 64, 24, Bp, C, D, E, None) == B.ERR_SHAPE


def test_linear_workspace_bytes(L):
    wb = L.nvfp4_linear_workspace_bytes
    assert wb(1, 5120, 5120) == 0            # GEMV: no workspace
    # prefill GEMM: K split only while the 128 x 272 tiles leave CUs idle (at most 128 tiles, or 257..384): the
    # counter region + slices x split tiles x 139,264-byte FP32 partial tiles
    assert wb(65, 17408, 5120) == 16384 + 4 * 64 * 139264        # 64 tiles, 4 slices
    assert wb(512, 5120, 17408) == 16384 + 3 * 76 * 139264       # 76 tiles, 3 slices
    assert wb(512, 17408, 5120) == 0                              # 256 tiles fill the chip
    assert wb(2048, 5120, 17408) == 16384 + 5 * 48 * 139264       # 304 tiles: 256 whole, 48 split in 5 slices
    assert wb(2048, 17408, 5120) == 0                             # 1024 tiles
    assert wb(65, 17408, 5136) == 0                               # K not a multiple of 256: other kernel
    assert wb(8, 17408, 5120) == 0           # small-M, 68 rows x 1 K slice per workgroup
    # small-M down projection: 64 blocks of 80 rows x 4 K slices; the fixed 16 KiB counter region + 4 * m * n
    # FP32 partials
    assert wb(8, 5120, 17408) == 16384 + 4 * 8 * 5120 * 4
    assert wb(32, 5120, 17408) == 16384 + 4 * 32 * 5120 * 4
    assert wb(-1, 64, 64) == -1 and wb(8, 64, 24) == -1 and wb(8, 0, 64) == -1


def test_linear_ws_validation(L):
    lw = L.nvfp4_linear_ws
    W = 0x60000000
    assert lw(A, 8, 64, 64, Bp, C, D, E, W, -1, None) == B.ERR_SHAPE     # negative workspace size
    assert lw(A, 8, 64, 64, Bp, C, D, E, W + 8, 1024, None) == B.ERR_ALIGN
    assert lw(A, 8, 64, 64, Bp, C, D, E, A + 64, 1024, None) == B.ERR_ALIAS   # overlaps x
    assert lw(A, 8, 64, 64, Bp, C, D, E, E - 512, 1024, None) == B.ERR_ALIAS  # overlaps y
    assert lw(A, 8, 64, 24, Bp, C, D, E, W, 1024, None) == B.ERR_SHAPE
    assert lw(None, 8, 64, 64, Bp, C, D, E, W, 1024, None) == B.ERR_NULL
    assert lw(None, 0, 64, 64, Bp, C, D, None, None, 0, None) == B.OK    # m = 0 no-op


def test_quantize_validation(L):
    q = L.nvfp4_quantize
    assert q(None, 4, 64, Bp, C, D, None) == B.ERR_NULL
    assert q(A, 4, 40, Bp, C, D, None) == B.ERR_SHAPE
    assert q(A, 0, 64, Bp, C, D, None) == B.ERR_SHAPE
    assert q(A, 4, 64, Bp + 1, C, D, None) == B.ERR_ALIGN
    assert q(A, 4, 64, A + 64, C, D, None) == B.ERR_ALIAS               # packed overlaps w (512 bytes)
    assert q(A, 4, 64, Bp, Bp + 64, D, None) == B.ERR_ALIAS             # scales overlaps packed (128 bytes)
    assert q(A, 4, 64, Bp, C, C, None) == B.ERR_ALIAS                   # tscale overlaps scales
    qa = L.nvfp4_quantize_with_amax
    assert qa(A, 4, 64, None, Bp, C, D, None) == B.ERR_NULL
    assert qa(A, 4, 64, E + 4, Bp, C, D, None) == B.ERR_ALIGN
    assert qa(A, 4, 64, D, Bp, C, D, None) == B.ERR_ALIAS               # amax overlaps tscale
    am = L.nvfp4_amax_accumulate
    assert am(A, 4, 64, None, None) == B.ERR_NULL
    assert am(A, 4, 48 + 1, E, None) == B.ERR_SHAPE
    assert am(A, 4, 64, A + 32, None) == B.ERR_ALIAS


def test_dequant_validation(L):
    dq = L.nvfp4_dequant
    assert dq(None, C, D, 4, 64, E, None) == B.ERR_NULL
    assert dq(A, C, D, 4, 8, E, None) == B.ERR_SHAPE
    assert dq(A, C, D, 4, 64, E + 2, None) == B.ERR_ALIGN
    assert dq(A, C, D, 4, 64, A, None) == B.ERR_ALIAS


def test_grouped_workspace_bytes(L):
    wb = L.nvfp4_linear_grouped_workspace_bytes
    # int32 cnt[e], pair_off[e + 1], tile_off[e + 1], perm[t * topk], rounded up to 16 bytes
    assert wb(10, 8, 128) == 1872           # (3 * 128 + 2 + 80) * 4 = 1864 -> 1872
    assert wb(0, 1, 1) == 32                # (3 + 2) * 4 = 20 -> 32
    assert wb(4096, 8, 128) == 132624        # (3 * 128 + 2 + 32768) * 4 = 132616 -> 132624
    assert wb(-1, 1, 1) == -1 and wb(1, 0, 1) == -1 and wb(1, 1, 0) == -1
    assert wb(2 ** 62, 4, 1) == -1           # t * topk overflows


def test_grouped_validation(L):
    g = L.nvfp4_linear_grouped
    R, W = 0x60000000, 0x70000000
    need = L.nvfp4_linear_grouped_workspace_bytes(2, 2, 2)
    args = lambda x=A, t=2, topk=2, e=2, y=E, ws=W, wsb=need: (x, t, topk, R, e, 64, 256, Bp, C, D, y, ws,  # noqa: E731
                                                                 wsb, None)
    assert g(*args(ws=None)) == B.ERR_NULL
    assert g(*args(wsb=need - 16)) == B.ERR_SHAPE
    assert g(*args(topk=0)) == B.ERR_SHAPE and g(*args(e=0)) == B.ERR_SHAPE
    assert g(*args(ws=W + 8)) == B.ERR_ALIGN
    assert g(*args(ws=A + 64)) == B.ERR_ALIAS      # workspace overlaps x
    assert g(*args(ws=E + 16)) == B.ERR_ALIAS      # workspace overlaps y
    assert g(*args(ws=R)) == B.ERR_ALIAS           # workspace overlaps route
    assert g(*args(y=A + 32)) == B.ERR_ALIAS       # y overlaps x
    assert g(*args(x=None, t=0, y=None, ws=None, wsb=0)) == B.OK    # t = 0 no-op


def test_kv_gather_validation(L):
    g = L.nvfp4_kv_gather
    BT, SL, DS, O = 0x60000000, 0x61000000, 0x62000000, 0x70000000

    def args(fmt=0, out=0, codes=A, scales=Bp, ts=D, nb=4, bs=16, heads=2, hd=64, mb=3, seqs=2, o=O, rows=100):
        return (fmt, out, codes, scales, ts, nb, bs, heads, hd, BT, mb, SL, DS, seqs, o, rows, None)
    assert g(*args(fmt=2)) == B.ERR_UNSUPPORTED and g(*args(out=2)) == B.ERR_UNSUPPORTED
    assert g(*args(codes=None)) == B.ERR_NULL
    assert g(*args(ts=None)) == B.ERR_NULL                        # NVFP4 needs its tensor scale
    assert g(*args(hd=24)) == B.ERR_SHAPE                         # head_dim % 16 != 0
    assert g(*args(fmt=1, hd=48, ts=None)) == B.ERR_SHAPE         # MXFP4: head_dim % 32 != 0
    assert g(*args(bs=0)) == B.ERR_SHAPE and g(*args(nb=0)) == B.ERR_SHAPE and g(*args(mb=0)) == B.ERR_SHAPE
    assert g(*args(seqs=-1)) == B.ERR_SHAPE and g(*args(rows=-1)) == B.ERR_SHAPE
    assert g(*args(seqs=2 ** 20, mb=2 ** 12)) == B.ERR_SHAPE        # 2^32 workgroups
    assert g(*args(codes=A + 8)) == B.ERR_ALIGN and g(*args(o=O + 8)) == B.ERR_ALIGN
    assert g(*args(o=A)) == B.ERR_ALIAS                           # out overlaps the codes
    assert g(*args(seqs=0)) == B.OK                               # no-op


def test_mx_validation(L):
    W = 0x70000000
    q, d, g, lw, wb = L.nvfp4_mx_quantize, L.nvfp4_mx_dequant, L.nvfp4_mx_gemm, L.nvfp4_mx_linear_w4a4, \
        L.nvfp4_mx_linear_w4a4_workspace_bytes
    assert q(A, 4, 48, Bp, C, None) == B.ERR_SHAPE                      # k % 32 != 0
    assert q(A, 0, 64, None, None, None) == B.OK                         # rows = 0 no-op
    assert q(None, 4, 64, Bp, C, None) == B.ERR_NULL
    assert q(A + 8, 4, 64, Bp, C, None) == B.ERR_ALIGN
    assert q(A, 4, 64, A + 64, C, None) == B.ERR_ALIAS                   # packed overlaps w
    assert d(Bp, C, 4, 64, Bp + 16, None) == B.ERR_ALIAS
    assert g(A, Bp, 8, C, D, 64, 320, E, None) == B.ERR_UNSUPPORTED      # k % 256 != 0
    assert g(A, Bp, 8, C, D, 0, 512, E, None) == B.ERR_SHAPE             # n = 0
    assert g(A, Bp, 0, C, D, 64, 512, None, None) == B.OK                # m = 0 no-op
    assert g(A, Bp, 8, C, D, 64, 512, A + 16, None) == B.ERR_ALIAS       # y overlaps xq
    assert wb(8, 512) == 8 * 256 + 8 * 16 and wb(3, 32) == 48 + 16 and wb(8, 48) == -1
    assert lw(A, 8, 64, 512, C, D, E, W, wb(8, 512) - 16, None) == B.ERR_SHAPE   # workspace too small
    assert lw(A, 8, 64, 512, C, D, E, None, wb(8, 512), None) == B.ERR_NULL
    assert lw(A, 8, 64, 512, C, D, E, A, wb(8, 512), None) == B.ERR_ALIAS       # workspace overlaps x
    assert lw(A, 8, 64, 320, C, D, E, W, wb(8, 320), None) == B.ERR_UNSUPPORTED


def test_linear_w4a4_validation(L):
    f, wb = L.nvfp4_linear_w4a4, L.nvfp4_linear_w4a4_workspace_bytes
    W = 0x70000000
    # codes 8*256 | scales 8*32 | 16 bytes of floats | decoded 8*512*2
    assert wb(8, 512) == 8 * 256 + 8 * 32 + 16 + 8 * 512 * 2
    assert wb(3, 48) == 80 + 16 + 16 + 3 * 48 * 2       # 72 and 9 bytes rounded up to 16
    assert wb(0, 512) == 0 and wb(8, 40) == -1 and wb(-1, 512) == -1
    n = 64
    need = wb(8, 512)
    assert f(A, 0, n, 512, C, D, E, None, None, 0, None) == B.OK                      # m = 0 no-op
    assert f(A, 8, n, 40, C, D, E, E, W, need, None) == B.ERR_SHAPE                 # k % 16 != 0
    assert f(A, 8, n, 512, C, D, E, E + 4096, None, need, None) == B.ERR_NULL
    assert f(A, 8, n, 512, C, D, E, E + 4096, W, need - 16, None) == B.ERR_SHAPE   # workspace too small
    assert f(A, 8, n, 512, C, D, E, E + 4096, W, -1, None) == B.ERR_SHAPE
    assert f(A, 8, n, 512, C, D, E, E + 4096, W + 8, need, None) == B.ERR_ALIGN
    assert f(A, 8, n, 512, C, D, E, E + 4096, A + 16, need, None) == B.ERR_ALIAS   # workspace overlaps x
    assert f(A, 8, n, 512, C, D, E, E + 4096, C, need, None) == B.ERR_ALIAS        # overlaps packed
    assert f(A, 8, n, 512, C, D, E, A, W, need, None) == B.ERR_ALIAS                # y overlaps x


def test_binding_workspace_kept_when_superseded_and_refused_under_capture(monkeypatch):
    """The binding's per-stream split-K workspace: a larger shape replaces it without freeing the old one
    (a captured graph may still point at it), and no workspace is created while a capture is running."""
    import torch

    monkeypatch.setattr(B, "_workspaces", {})
    monkeypatch.setattr(B, "_superseded", [])
    capturing = {"on": False}
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: capturing["on"])
    dev = torch.device("cpu", 0)
    a = B._workspace_for(dev, 7, 1000)
    assert a.numel() == 1000 and not a.any()
    assert B._workspace_for(dev, 7, 800) is a                   # big enough: reused as is
    b = B._workspace_for(dev, 7, 1500)                          # grows geometrically
    assert b.numel() == 2000 and B._superseded == [a]           # the old one stays referenced
    capturing["on"] = True
    assert B._workspace_for(dev, 7, 2000) is b                  # an existing one may be used in a capture
    with pytest.raises(RuntimeError, match="graph capture"):
        B._workspace_for(dev, 7, 4000)                          # but none is allocated there
    with pytest.raises(RuntimeError, match="graph capture"):
        B._workspace_for(dev, 8, 16)                            # nor for a new stream
    capturing["on"] = False
    q = B._workspace_for(dev, 7, 4096, kind="quantize")         # the quantizer's partial maxima: its own buffer,
    assert q is not b and B._workspace_for(dev, 7, 16) is b     # never the counters of the split workspace


def test_linear_noalloc_validation(L):
    f = L.nvfp4_linear_noalloc
    assert L.nvfp4_linear_noalloc_max_bytes() == 8 << 20
    # every split the small-M kernel plans for m <= 64 fits the library's scratch
    for m in (2, 8, 32, 64):
        for n in (16, 300, 1280, 5120, 13651, 17408):
            for k in (256, 4096, 17408):
                assert 0 <= L.nvfp4_linear_workspace_bytes(m, n, k) <= L.nvfp4_linear_noalloc_max_bytes()
    assert f(None, 8, 64, 64, Bp, C, D, E, None) == B.ERR_NULL
    assert f(A, 8, 64, 24, Bp, C, D, E, None) == B.ERR_SHAPE          # k % 16 != 0
    assert f(A, -1, 64, 64, Bp, C, D, E, None) == B.ERR_SHAPE         # m < 0
    assert f(A + 8, 8, 64, 64, Bp, C, D, E, None) == B.ERR_ALIGN
    assert f(A, 8, 64, 64, Bp, C, D, A + 16, None) == B.ERR_ALIAS     # y overlaps x
    assert f(None, 0, 64, 64, Bp, C, D, None, None) == B.OK           # m = 0 no-op


def test_prepared_layout_validation(L):
    pb = L.nvfp4_prepared_bytes
    assert pb(16, 128) == 1152 and pb(17, 256) == 2 * 2 * 1152 and pb(17408, 5120) == 17408 * 5120 * 9 // 16
    assert pb(16, 96) == -1 and pb(0, 128) == -1 and pb(16, 0) == -1
    p = L.nvfp4_prepare
    assert p(None, C, 16, 128, E, None) == B.ERR_NULL
    assert p(Bp, C, 16, 96, E, None) == B.ERR_SHAPE            # k % 128 != 0
    assert p(Bp + 8, C, 16, 128, E, None) == B.ERR_ALIGN
    assert p(Bp, C, 16, 128, Bp + 512, None) == B.ERR_ALIAS     # output overlaps packed
    d = L.nvfp4_dequant_prepared
    assert d(None, D, 16, 128, E, None) == B.ERR_NULL
    assert d(Bp, D, 16, 64, E, None) == B.ERR_SHAPE
    assert d(Bp, D, 16, 128, Bp + 16, None) == B.ERR_ALIAS
    wb = L.nvfp4_linear_prepared_workspace_bytes
    assert wb(8, 64, 96) == -1 and wb(-1, 64, 128) == -1 and wb(0, 64, 128) == 0 and wb(33, 64, 128) == 0
    # down projection: 64 blocks of 80 rows x 4 K slices (the fixed 16 KiB counter region + 4 * m * n FP32
    # partials); up projection: 68 rows x 1 slice, no workspace
    assert wb(8, 5120, 17408) == 16384 + 4 * 8 * 5120 * 4 and wb(8, 17408, 5120) == 0
    lp = L.nvfp4_linear_prepared
    assert lp(None, 8, 64, 128, Bp, D, E, None, 0, None) == B.ERR_NULL
    assert lp(A, 8, 64, 96, Bp, D, E, None, 0, None) == B.ERR_SHAPE
    assert lp(A, 33, 64, 128, Bp, D, E, None, 0, None) == B.ERR_UNSUPPORTED   # prefill m
    assert lp(A + 8, 8, 64, 128, Bp, D, E, None, 0, None) == B.ERR_ALIGN
    assert lp(A, 8, 64, 128, Bp, D, A + 16, None, 0, None) == B.ERR_ALIAS    # y overlaps x
    assert lp(None, 0, 64, 128, Bp, D, None, None, 0, None) == B.OK          # m = 0 no-op


def test_quantize_ws_validation(L):
    q = L.nvfp4_quantize_ws
    W = 0x70000000
    assert L.nvfp4_quantize_workspace_bytes() == 4096
    assert q(None, 16, 32, Bp, C, D, W, 4096, None) == B.ERR_NULL
    assert q(A, 16, 30, Bp, C, D, W, 4096, None) == B.ERR_SHAPE
    assert q(A, 16, 32, Bp, C, D, W, -1, None) == B.ERR_SHAPE
    assert q(A, 16, 32, Bp, C, D, W + 8, 4096, None) == B.ERR_ALIGN
    assert q(A, 16, 32, Bp, C, D, A + 16, 4096, None) == B.ERR_ALIAS      # workspace overlaps w
    assert q(A, 16, 32, Bp, C, D, D, 4096, None) == B.ERR_ALIAS           # workspace overlaps tscale
    assert q(A, 16, 32, Bp + 8, C, D, W, 4096, None) == B.ERR_ALIGN
    assert q(A, 16, 32, Bp + 8, C, D, W + 8, 4095, None) == B.ERR_ALIGN    # too small: nvfp4_quantize's checks


def test_stream_read_validation(L):
    f = L.nvfp4_stream_read
    assert f(None, 1024, E, None) == B.ERR_NULL
    assert f(A, 1000, E, None) == B.ERR_SHAPE and f(A, 0, E, None) == B.ERR_SHAPE
    assert f(A + 8, 1024, E, None) == B.ERR_ALIGN
    assert f(A, 1024, A + 16, None) == B.ERR_ALIAS
    w = L.nvfp4_stream_read_sink_words
    assert w(0) == -1 and w(1000) == -1
    assert w(16) == 1 and w(16 * 2048) == 1 and w(16 * 2048 + 16) == 2      # 2048 16-byte loads per workgroup
    assert w(1 << 40) == 8192
