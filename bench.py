"""Benchmark of the NVFP4 W4A16 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the decode GEMV (M = 1, N = K = 5120, BF16 ~N(0, 0.02) weights with
1% outlier input columns x8, RTN-quantized to NVFP4; BF16 ~N(0, 1)
activations).  A step is one call of the decode hot path, nvfp4_linear at
M = 1 (GEMV + BF16 epilogue), on one of 37 rotated weight copies (the rotated
set is 2x the 256 MB Infinity Cache, so every call streams its weights from
HBM).  The K timed calls are replayed from a HIP graph of the rotated launch
sequence, bracketed by HIP events on the stream they run on.

The same run also measures every other row of the hot path once each
(quantizer, dequantizer, merged gate/up GEMV, small-M batched decode, prefill
GEMM) and reports them under "rows"; it times the CPU oracle on a bounded
sample as a baseline ("cpu_baseline").  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import nvfp4_weight_only_amd as nv  # noqa: E402
from nvfp4_weight_only_amd import workloads as WL  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published (no sparsity)
INFINITY_CACHE = 256 << 20


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def linear_bytes(m, n, k):
    """Algorithmic HBM bytes of one linear call: packed + scales + X + Y + tensor scale."""
    return n * k // 2 + n * k // 16 + 2 * m * k + 2 * m * n + 4


def copies_needed(bytes_per_copy):
    return max(2, -(-2 * INFINITY_CACHE // bytes_per_copy))


class Rotated:
    """C rotated copies of one quantized weight (distinct HBM addresses)."""

    def __init__(self, packed, scales, tscale, c):
        self.items = [(packed.clone(), scales.clone(), tscale.clone()) for _ in range(c)]

    def __len__(self):
        return len(self.items)


def graph_of(calls):
    """Capture a list of zero-argument launch closures into one HIP graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:          # warm once outside the graph on the capture stream
            c()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def warm_graph(graph, seconds=0.1):
    """Replay until `seconds` of wall time have passed: the clocks settle at their loaded state first."""
    t_end = time.perf_counter() + seconds
    while True:
        graph.replay()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            return


def time_graph_replays(graph, replays, launches_per_replay):
    """Average duration per launch (ms) over `replays` back-to-back graph replays, by HIP events."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * launches_per_replay)


def linear_calls(x, rot, y, kernel="auto"):
    return [(lambda p=p, s=s, t=t: nv.linear(x, p, s, t, kernel=kernel, out=y)) for (p, s, t) in rot.items]


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "nvfp4_weight_only_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches the current source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    e = table.get(kernel_key)
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# Rows of the hot path.
# ---------------------------------------------------------------------------
def bench_linear_row(wname, m, reps, kernel="auto"):
    wl = WL.WORKLOADS[wname]
    w = wl.weight()
    packed, scales, tscale = nv.quantize(dev_bf16(w))
    del w
    per_copy = packed.numel() + scales.numel()
    rot = Rotated(packed, scales, tscale, copies_needed(per_copy))
    x = dev_bf16(wl.activations(m))
    y = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
    g = graph_of(linear_calls(x, rot, y, kernel))
    warm_graph(g)
    ms = time_graph_replays(g, reps, len(rot))
    nbytes = linear_bytes(m, wl.n, wl.k)
    flops = 2.0 * m * wl.n * wl.k
    out = {"m": m, "n": wl.n, "k": wl.k, "copies": len(rot), "us_per_call": round(ms * 1e3, 3),
           "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "tflop_s": round(flops / (ms * 1e-3) / 1e12, 2),
           "weight_streams_per_s": round(1.0 / (ms * 1e-3), 1)}
    out["hbm_frac"] = round(out["gb_s"] / HBM_PEAK_GBS, 4)
    out["mfma_frac"] = round(out["tflop_s"] / BF16_MFMA_PEAK_TFLOPS, 4)
    del rot, g
    torch.cuda.empty_cache()
    return out


def bench_prepared_row(wname, m, reps):
    """nvfp4_linear_prepared on the kernel-native layout of the workload's weight, rotated copies (the same
    algorithmic bytes as the checkpoint layout: the layout is a permutation of them)."""
    wl = WL.WORKLOADS[wname]
    packed, scales, tscale = nv.quantize(dev_bf16(wl.weight()))
    prep = nv.prepare(packed, scales)
    del packed, scales
    c = copies_needed(prep.numel())
    items = [(prep.clone(), tscale.clone()) for _ in range(c)]
    del prep
    x = dev_bf16(wl.activations(m))
    y = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
    calls = [(lambda p=p, t=t: nv.linear_prepared(x, p, t, wl.n, out=y)) for (p, t) in items]
    g = graph_of(calls)
    warm_graph(g)
    ms = time_graph_replays(g, reps, len(items))
    nbytes = linear_bytes(m, wl.n, wl.k)
    flops = 2.0 * m * wl.n * wl.k
    out = {"m": m, "n": wl.n, "k": wl.k, "copies": c, "layout": "kernel-native (nvfp4_prepare)",
           "us_per_call": round(ms * 1e3, 3), "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "tflop_s": round(flops / (ms * 1e-3) / 1e12, 2), "weight_streams_per_s": round(1.0 / (ms * 1e-3), 1)}
    out["hbm_frac"] = round(out["gb_s"] / HBM_PEAK_GBS, 4)
    out["mfma_frac"] = round(out["tflop_s"] / BF16_MFMA_PEAK_TFLOPS, 4)
    del items, g
    torch.cuda.empty_cache()
    return out


def bench_prepare_row(reps):
    """nvfp4_prepare (checkpoint -> kernel-native layout) of the small-M up weight: read and write 0.5625 B per
    element each."""
    wl = WL.WORKLOADS["small_m_up"]
    packed, scales, _ = nv.quantize(dev_bf16(wl.weight()))
    c = copies_needed(2 * (packed.numel() + scales.numel()))
    items = [(packed.clone(), scales.clone(), torch.empty(nv.prepared_bytes(wl.n, wl.k), dtype=torch.uint8,
                                                           device="cuda")) for _ in range(c)]
    L = nv.lib()

    def call(p, s, o):
        L.nvfp4_prepare(p.data_ptr(), s.data_ptr(), wl.n, wl.k, o.data_ptr(), torch.cuda.current_stream().cuda_stream)

    g = graph_of([(lambda it=it: call(*it)) for it in items])
    warm_graph(g)
    ms = time_graph_replays(g, reps, len(items))
    nbytes = 2 * (packed.numel() + scales.numel())
    return {"n": wl.n, "k": wl.k, "copies": c, "us_per_call": round(ms * 1e3, 3),
            "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def bench_stream_rows(reps):
    """Plain streaming reads (nvfp4_stream_read) of the weight sizes the linear streams: the measured HBM read
    rate the other rows are also reported against."""
    out = {}
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    L = nv.lib()
    for name, nbytes in (("decode", 14_766_080), ("small_m", 50_495_488), ("gate_up", 100_352_000)):
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies_needed(nbytes))]
        for b in bufs:
            b.fill_(1)

        def call(b):
            L.nvfp4_stream_read(b.data_ptr(), nbytes, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)

        g = graph_of([(lambda b=b: call(b)) for b in bufs])
        warm_graph(g)
        ms = time_graph_replays(g, reps, len(bufs))
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"stream_read_{name}_{nbytes}B"] = {"bytes": nbytes, "copies": len(bufs), "us_per_call": round(ms * 1e3, 3),
                                                "gb_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        del bufs, g
        torch.cuda.empty_cache()
    return out


def bench_quant_rows(reps):
    """Quantizer (amax + encode passes; with and without a workspace) and dequantizer on the decode weight,
    rotated."""
    wl = WL.WORKLOADS["decode"]
    w = dev_bf16(wl.weight())
    n, k = wl.n, wl.k
    c = copies_needed(2 * n * k)
    ws = [w.clone() for _ in range(c)]
    outs = [nv.quantize(wi) for wi in ws]
    g = graph_of([(lambda wi=wi: nv.quantize(wi)) for wi in ws])          # nvfp4_quantize_ws: 2 launches
    warm_graph(g)
    ms_q = time_graph_replays(g, reps, c)
    g3 = graph_of([(lambda wi=wi: nv.quantize(wi, workspace=None)) for wi in ws])   # nvfp4_quantize: 3 launches
    warm_graph(g3)
    ms_q3 = time_graph_replays(g3, reps, c)
    del g3
    dq = [torch.empty((n, k), dtype=torch.bfloat16, device="cuda") for _ in range(c)]
    lib = nv.lib()

    def dq_call(o, d):
        return lambda: lib.nvfp4_dequant(o[0].data_ptr(), o[1].data_ptr(), o[2].data_ptr(), n, k, d.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)
    g2 = graph_of([dq_call(o, d) for o, d in zip(outs, dq)])
    warm_graph(g2)
    ms_d = time_graph_replays(g2, reps, c)
    e = n * k
    q_bytes = 2 * e + 2 * e + e // 2 + e // 16 + 4     # amax read, quantize read, packed + scales write
    d_bytes = e // 2 + e // 16 + 4 + 2 * e
    rows = {
        "quantize_decode_5120x5120": {"us_per_call": round(ms_q * 1e3, 2),
                                      "gb_s": round(q_bytes / (ms_q * 1e-3) / 1e9, 1),
                                      "hbm_frac": round(q_bytes / (ms_q * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                      "bytes": q_bytes,
                                      "note": "nvfp4_quantize_ws, 2 launches: per-workgroup amax (at most 1024 "
                                              "partial maxima), then the encode pass, each workgroup of which "
                                              "reduces the partial maxima itself"},
        "quantize_3launch_decode_5120x5120": {"us_per_call": round(ms_q3 * 1e3, 2),
                                              "gb_s": round(q_bytes / (ms_q3 * 1e-3) / 1e9, 1),
                                              "hbm_frac": round(q_bytes / (ms_q3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                              "bytes": q_bytes,
                                              "note": "nvfp4_quantize (no workspace): amax, tensor scale, encode"},
        "dequant_decode_5120x5120": {"us_per_call": round(ms_d * 1e3, 2),
                                     "gb_s": round(d_bytes / (ms_d * 1e-3) / 1e9, 1),
                                     "hbm_frac": round(d_bytes / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                     "bytes": d_bytes},
    }
    del ws, outs, dq, g, g2
    torch.cuda.empty_cache()
    return rows


def bench_moe_rows(reps):
    """Routed MoE rows over one 128-expert stack (N=2048, K=4096):
    decode: nvfp4_linear_routed, one token, over a rotation of routes that reads every expert once;
    prefill: nvfp4_linear_grouped, 2048 tokens routed top-8 by a balanced random router (the whole call:
             grouping kernels and the grouped GEMM)."""
    mw = WL.MOE_DECODE
    base = dev_bf16(mw.base_weight())
    stack = torch.stack([(base.float() * mw.expert_scale(i)).to(torch.bfloat16) for i in range(mw.experts)])
    del base
    packed, scales, tscale = nv.quantize_experts(stack)
    del stack
    torch.cuda.empty_cache()
    w_bytes = mw.n * mw.k // 2 + mw.n * mw.k // 16 + 4
    rows = {}

    routes = [torch.from_numpy(r).cuda() for r in mw.routes()]
    x = dev_bf16(WL.activations(mw.t, mw.k))
    y = torch.empty((mw.t, mw.topk, mw.n), dtype=torch.bfloat16, device="cuda")
    calls = [(lambda r=r: nv.linear_routed(x, r, packed, scales, tscale, out=y)) for r in routes]
    g = graph_of(calls)
    warm_graph(g)
    ms = time_graph_replays(g, reps, len(calls))
    nbytes = mw.t * mw.topk * (w_bytes + 2 * mw.n) + 2 * mw.t * mw.k + 4 * mw.t * mw.topk
    flops = 2.0 * mw.t * mw.topk * mw.n * mw.k
    row = {"experts": mw.experts, "n": mw.n, "k": mw.k, "topk": mw.topk, "tokens": mw.t, "routes": len(calls),
           "us_per_call": round(ms * 1e3, 3), "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "tflop_s": round(flops / (ms * 1e-3) / 1e12, 2), "bytes": nbytes}
    row["hbm_frac"] = round(row["gb_s"] / HBM_PEAK_GBS, 4)
    rows["moe_routed_decode_top8"] = row
    del g, routes, x, y

    pw = WL.MOE_PREFILL
    route = torch.from_numpy(pw.random_routes()).cuda()
    x = dev_bf16(WL.activations(pw.t, pw.k))
    y = torch.empty((pw.t, pw.topk, pw.n), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(nv.linear_grouped_workspace_bytes(pw.t, pw.topk, pw.experts), dtype=torch.uint8, device="cuda")
    g = graph_of([lambda: nv.linear_grouped(x, route, packed, scales, tscale, out=y, workspace=ws)])
    warm_graph(g)
    ms = time_graph_replays(g, max(reps // 3, 3), 1)
    pairs = pw.t * pw.topk
    flops = 2.0 * pairs * pw.n * pw.k
    nbytes = pw.experts * w_bytes + 2 * pw.t * pw.k + 2 * pairs * pw.n + 4 * pairs
    row = {"experts": pw.experts, "n": pw.n, "k": pw.k, "topk": pw.topk, "tokens": pw.t,
           "pairs_per_expert": [int(c) for c in torch.bincount(route.flatten().long(), minlength=pw.experts)
                                .aminmax()],
           "us_per_call": round(ms * 1e3, 3), "tflop_s": round(flops / (ms * 1e-3) / 1e12, 2),
           "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes}
    row["mfma_frac"] = round(row["tflop_s"] / BF16_MFMA_PEAK_TFLOPS, 4)
    rows["moe_grouped_prefill_t2048_top8"] = row
    del g, route, x, y, ws, packed, scales, tscale
    torch.cuda.empty_cache()
    return rows


def bench_kv_rows(reps):
    """Paged FP4 KV-cache gather (nvfp4_kv_gather) on the chunked-prefill workload: 16 sequences, 66,971 past
    tokens of 8 heads x 128 in 16-token pages, to FP16; rotated cache + output copies."""
    kw = WL.KV_PREFILL
    table, lens, dst, nb, out_rows = kw.layout()
    tokens = int(lens.sum())
    elems = tokens * kw.heads * kw.head_dim
    td, ld, dd = (torch.from_numpy(a).cuda() for a in (table, lens, dst))
    rows = {}
    for fmt in ("nvfp4", "mxfp4"):
        codes, scales = kw.cache(fmt, nb)
        cd, sd = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
        ts = torch.tensor([kw.KV_TSCALE], dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None
        per_copy = cd.numel() + sd.numel() + 2 * out_rows * kw.heads * kw.head_dim
        c = copies_needed(per_copy)
        items = [(cd.clone(), sd.clone(),
                  torch.zeros((out_rows, kw.heads, kw.head_dim), dtype=torch.float16, device="cuda"))
                 for _ in range(c)]
        calls = [(lambda i=i: nv.kv_gather(i[0], i[1], ts, td, ld, dd, i[2], fmt=fmt)) for i in items]
        g = graph_of(calls)
        warm_graph(g)
        ms = time_graph_replays(g, reps, len(calls))
        nbytes = elems // 2 + elems // (16 if fmt == "nvfp4" else 32) + 2 * elems
        row = {"format": fmt, "out": "f16", "seqs": kw.seqs, "tokens": tokens, "heads": kw.heads,
               "head_dim": kw.head_dim, "block_size": kw.block_size, "copies": c,
               "us_per_call": round(ms * 1e3, 3), "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes}
        row["hbm_frac"] = round(row["gb_s"] / HBM_PEAK_GBS, 4)
        rows[f"kv_gather_{fmt}_f16"] = row
        del g, items, cd, sd
        torch.cuda.empty_cache()
    return rows


FP4_MFMA_PEAK_TFLOPS = 10066.3  # MI355X dense FP4 / FP6 MFMA, published (no sparsity)


def bench_mx_rows(reps):
    """W4A4 MXFP4 linear (nvfp4_mx_linear_w4a4: X quantized to MXFP4 on the stream, then the FP4 GEMM) on the
    prefill workload (N=17408, K=5120) at M=512 and 2048, rotated weight copies; also the GEMM alone."""
    wl = WL.WORKLOADS["prefill"]
    wq, wsc = nv.mx_quantize(dev_bf16(wl.weight()))
    c = copies_needed(wq.numel() + wsc.numel())
    rot = [(wq.clone(), wsc.clone()) for _ in range(c)]
    rows = {}
    for m in (512, 2048):
        x = dev_bf16(wl.activations(m))
        y = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(nv.lib().nvfp4_mx_linear_w4a4_workspace_bytes(m, wl.k), dtype=torch.uint8, device="cuda")
        g = graph_of([(lambda r=r: nv.mx_linear_w4a4(x, r[0], r[1], out=y, workspace=ws)) for r in rot])
        warm_graph(g)
        ms = time_graph_replays(g, reps, len(rot))
        xq, xs = nv.mx_quantize(x)
        g2 = graph_of([(lambda r=r: nv.mx_gemm(xq, xs, r[0], r[1], out=y)) for r in rot])
        warm_graph(g2)
        ms_g = time_graph_replays(g2, reps, len(rot))
        flops = 2.0 * m * wl.n * wl.k
        row = {"m": m, "n": wl.n, "k": wl.k, "copies": c, "us_per_call": round(ms * 1e3, 3),
               "tflop_s": round(flops / (ms * 1e-3) / 1e12, 1), "gemm_us": round(ms_g * 1e3, 3),
               "gemm_tflop_s": round(flops / (ms_g * 1e-3) / 1e12, 1)}
        row["fp4_frac"] = round(row["tflop_s"] / FP4_MFMA_PEAK_TFLOPS, 4)
        row["gemm_fp4_frac"] = round(row["gemm_tflop_s"] / FP4_MFMA_PEAK_TFLOPS, 4)
        rows[f"mx_w4a4_prefill_m{m}"] = row
        del g, g2
    del rot
    torch.cuda.empty_cache()
    return rows


def bench_w4a4_nvfp4_row(m, reps):
    """NVFP4 x NVFP4 linear (nvfp4_linear_w4a4: X quantized to NVFP4 on the stream, decoded exactly to BF16, then
    the BF16-MFMA GEMM) on the prefill workload (N=17408, K=5120), rotated weight copies."""
    wl = WL.WORKLOADS["prefill"]
    packed, scales, tscale = nv.quantize(dev_bf16(wl.weight()))
    rot = Rotated(packed, scales, tscale, copies_needed(packed.numel() + scales.numel()))
    x = dev_bf16(wl.activations(m))
    y = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(nv.linear_w4a4_workspace_bytes(m, wl.k), dtype=torch.uint8, device="cuda")
    g = graph_of([(lambda p=p, s=s, t=t: nv.linear_w4a4(x, p, s, t, out=y, workspace=ws)) for (p, s, t) in rot.items])
    warm_graph(g)
    ms = time_graph_replays(g, reps, len(rot))
    flops = 2.0 * m * wl.n * wl.k
    row = {"m": m, "n": wl.n, "k": wl.k, "copies": len(rot), "us_per_call": round(ms * 1e3, 3),
           "tflop_s": round(flops / (ms * 1e-3) / 1e12, 1)}
    row["mfma_frac"] = round(row["tflop_s"] / BF16_MFMA_PEAK_TFLOPS, 4)
    del rot, g
    torch.cuda.empty_cache()
    return {f"nvfp4_w4a4_prefill_m{m}": row}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands (numpy, float64), timed on the host
# cores in a child process (fork after the data are built, no GPU there).
# ---------------------------------------------------------------------------
_CPU = {}   # the data of the configuration being timed, inherited by the forked workers

# (name, k, weight kind, activation rows of the linear calls); the weight rows are a bounded sample:
# the first rows of the workload's weight (plain ~N(0, 0.02), with the outlier columns for decode; for the
# merged gate/up weight a plain ~N(0, 0.02) stand-in, since its two halves are rescaled over the whole tensor).
CPU_CONFIGS = [("tiny", 256, 512, "plain", (1,)), ("decode", 5120, 5120, "outliers", (1,)),
               ("gate_up", 34816, 5120, "plain", (1,)), ("small_m_up", 17408, 5120, "plain", (8, 32)),
               ("small_m_down", 5120, 17408, "plain", (8, 32)), ("prefill", 17408, 5120, "plain", (512, 2048))]


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    _CPU["limits"] = threadpool_limits(limits=1)   # one thread per worker: the pool is the parallelism


def _cpu_task(args):
    from oracle import nvfp4_oracle as O
    op, r0, r1 = args
    d = _CPU
    if op == "quantize":
        O.quantize(d["w"][r0:r1])
    elif op == "dequant":
        O.dequant(d["p"][r0:r1], d["s"][r0:r1], d["t"])
    else:
        O.linear_ref(d["x"][op], d["p"][r0:r1], d["s"][r0:r1], d["t"])
    return r1 - r0


def _cpu_time_op(pool, op, rows_per_task, cores, budget_s):
    """Rounds of one task per worker until budget_s of wall time; returns (rows processed, seconds)."""
    tasks = [(op, i * rows_per_task, (i + 1) * rows_per_task) for i in range(cores)]
    rows, t0 = 0, time.perf_counter()
    while True:
        rows += sum(pool.map(_cpu_task, tasks))
        el = time.perf_counter() - t0
        if el >= budget_s:
            return rows, el


def cpu_baseline_run(budget_s=20.0):
    """The oracle's quantize, dequant and float64 linear per configuration on all usable host cores."""
    import multiprocessing
    cores = min(len(os.sched_getaffinity(0)), 16)
    model = "unknown"
    with open("/proc/cpuinfo") as f:
        for line in f:
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    ops = sum(2 + len(ms) for *_, ms in CPU_CONFIGS)
    per_op = budget_s / ops
    ctx = multiprocessing.get_context("fork")
    out = {}
    for name, n, k, kind, ms in CPU_CONFIGS:
        # rows per task: about 0.15 s of work each (quantize ~370 ns, dequant ~11 ns per element on one core)
        rq = max(1, min(-(-n // cores), 400_000 // k))
        rd = max(1, min(-(-n // cores), 15_000_000 // k))
        rl = {m: max(1, min(-(-n // cores), int(0.15 / (k * (10 + 0.5 * m) * 1e-9)))) for m in ms}
        wrows, rows = cores * rq, cores * max([rd, *rl.values()])
        w = WL.weight_with_outlier_columns(wrows, k) if kind == "outliers" else WL.weight_plain(wrows, k)
        # Dequant and linear inputs: uniform random codes and E4M3 scale bytes 0x28..0x48 (1/8 .. 8); the
        # oracle's cost does not depend on the values, and quantizing this many rows first would take minutes.
        rng = np.random.default_rng(8)
        p = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
        sc = rng.integers(0x28, 0x49, size=(rows, k // 16), dtype=np.uint8)
        _CPU.clear()
        _CPU.update(w=w, p=p, s=sc, t=np.float32(1.0 / 64), x={m: WL.activations(m, k) for m in ms})
        res = {"n": n, "k": k}
        with ctx.Pool(cores, initializer=_cpu_worker_init) as pool:
            r, el = _cpu_time_op(pool, "quantize", rq, cores, per_op)
            res["quantize_gb_s"] = round(r * k * (2 + 2 + 0.5625) / el / 1e9, 4)
            r, el = _cpu_time_op(pool, "dequant", rd, cores, per_op)
            res["dequant_gb_s"] = round(r * k * 2.5625 / el / 1e9, 4)
            for m in ms:
                r, el = _cpu_time_op(pool, m, rl[m], cores, per_op)
                nb = r * (k // 2 + k // 16 + 2 * m) + 2 * m * k + 4
                res[f"linear_m{m}_gb_s"] = round(nb / el / 1e9, 4)
                res[f"linear_m{m}_gflop_s"] = round(2.0 * m * r * k / el / 1e9, 3)
        out[name] = res
    head = out["decode"]["linear_m1_gb_s"]
    return {"value": head, "unit": "GB/s", "cores": cores, "kind": "oracle", "cpu_model": model,
            "sample": (f"oracle (numpy float64) on {cores} host cores (one worker process each, one BLAS thread): "
                       f"value = linear_ref at M=1 on the decode shape (K=5120); per_config times quantize "
                       f"(amax + codes of the first weight rows; GB/s on 4.5625 B/element), dequant (2.5625 B/element) and "
                       f"linear_ref (random codes, scales 1/8..8) on row samples of every configuration, about "
                       f"{per_op:.1f} s each"),
            "per_config": out}


def cpu_baseline(budget_s=20.0):
    """Runs cpu_baseline_run in a child process (this process has initialised the GPU, so it forks nothing)."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only", "--cpu-budget",
                        str(budget_s)], capture_output=True, text=True, check=True)
    return json.loads(r.stdout.strip().splitlines()[-1])


def profile_run(what, launches, wname="decode", m=1, graph=False):
    """A short, untimed run for hardware-counter passes (rocprofv3 --pmc): `launches` launches of one kernel.

    decode: nvfp4_linear on the decode workload, cycling through rotated weight copies so that every
            launch streams its weights from HBM;
    prefill / prefill2048: nvfp4_linear on the prefill workload (N=17408, K=5120) at M=512 / 2048,
            rotated weight copies;
    copy:   a plain 256 MiB device-to-device copy (torch's copy kernel), the calibration for the
            FETCH_SIZE / WRITE_SIZE counters (each launch moves exactly 256 MiB each way);
    moe_prefill: nvfp4_linear_grouped on the grouped MoE prefill workload (2048 tokens, top-8 of 128
            experts of N=2048, K=4096), one call per launch (the sort kernel and the grouped GEMM);
    kv_gather: nvfp4_kv_gather (NVFP4 pages to FP16) on the chunked-prefill gather workload, cycling
            through rotated cache + output copies;
    mx_w4a4: nvfp4_mx_linear_w4a4 on the prefill workload at M=2048 (X quantized to MXFP4, then the FP4
            GEMM), rotated MXFP4 weight copies;
    nvfp4_w4a4: nvfp4_linear_w4a4 on the prefill workload at M=2048 (X quantized to NVFP4 and decoded, then
            the BF16-MFMA GEMM), rotated weight copies;
    quantize: nvfp4_quantize of the decode workload's BF16 weight (5120 x 5120), rotated input copies;
    dequant: nvfp4_dequant of the decode workload's quantized weight (5120 x 5120), rotated copies;
    linear: nvfp4_linear on workload `wname` at M = `m` (e.g. small_m_up / small_m_down at M = 8 or 32,
            gate_up at M = 1), rotated weight copies, the workspace-backed call as the bench rows make it;
    prepared: nvfp4_linear_prepared on the kernel-native layout of workload `wname` at M = `m`, rotated copies;
    stream: nvfp4_stream_read of the byte count the linear of workload `wname` streams (packed + scales),
            rotated buffers.
    With `graph`, the launches are the rotated sequence captured in one HIP graph and replayed (after the 0.1 s
    warm-up the bench rows get), as the bench rows time them; otherwise one host launch each.
    """
    torch.cuda.set_device(0)
    calls = []               # one zero-argument launch per rotated copy
    if what == "dequant":
        packed, scales, tscale = nv.quantize(dev_bf16(WL.WORKLOADS["decode"].weight()))
        rot = Rotated(packed, scales, tscale, copies_needed(packed.numel() * 5))
        outs = [torch.empty((packed.shape[0], packed.shape[1] * 2), dtype=torch.bfloat16, device="cuda")
                for _ in range(2)]
        calls = [(lambda p=p, s=s, t=t, o=outs[i % 2]: nv.dequant(p, s, t, out=o))
                 for i, (p, s, t) in enumerate(rot.items)]
    elif what == "linear":
        wl = WL.WORKLOADS[wname]
        packed, scales, tscale = nv.quantize(dev_bf16(wl.weight()))
        rot = Rotated(packed, scales, tscale, copies_needed(packed.numel() + scales.numel()))
        x = dev_bf16(wl.activations(m))
        y = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
        calls = linear_calls(x, rot, y)
    elif what == "prepared":
        wl = WL.WORKLOADS[wname]
        packed, scales, tscale = nv.quantize(dev_bf16(wl.weight()))
        prep = nv.prepare(packed, scales)
        del packed, scales
        items = [(prep.clone(), tscale.clone()) for _ in range(copies_needed(prep.numel()))]
        x = dev_bf16(wl.activations(m))
        y = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
        calls = [(lambda p=p, t=t: nv.linear_prepared(x, p, t, wl.n, out=y)) for (p, t) in items]
    elif what == "stream":
        wl = WL.WORKLOADS[wname]
        nbytes = wl.n * wl.k // 2 + wl.n * wl.k // 16
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies_needed(nbytes))]
        sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
        L = nv.lib()
        calls = [(lambda b=b: L.nvfp4_stream_read(b.data_ptr(), nbytes, sink.data_ptr(),
                                                  torch.cuda.current_stream().cuda_stream)) for b in bufs]
    elif what == "quantize":
        w = dev_bf16(WL.WORKLOADS["decode"].weight())
        rot = [w.clone() for _ in range(copies_needed(w.numel() * 2))]
        calls = [(lambda w=w: nv.quantize(w)) for w in rot]
    elif what == "nvfp4_w4a4":
        wl = WL.WORKLOADS["prefill"]
        m = 2048
        packed, scales, tscale = nv.quantize(dev_bf16(wl.weight()))
        rot = Rotated(packed, scales, tscale, copies_needed(packed.numel() + scales.numel()))
        x = dev_bf16(wl.activations(m))
        y = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(nv.linear_w4a4_workspace_bytes(m, wl.k), dtype=torch.uint8, device="cuda")
        calls = [(lambda p=p, s=s, t=t: nv.linear_w4a4(x, p, s, t, out=y, workspace=ws)) for (p, s, t) in rot.items]
    elif what == "mx_w4a4":
        wl = WL.WORKLOADS["prefill"]
        m = 2048
        wq, wsc = nv.mx_quantize(dev_bf16(wl.weight()))
        rot = [(wq.clone(), wsc.clone()) for _ in range(copies_needed(wq.numel() + wsc.numel()))]
        x = dev_bf16(wl.activations(m))
        y = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(nv.lib().nvfp4_mx_linear_w4a4_workspace_bytes(m, wl.k), dtype=torch.uint8, device="cuda")
        calls = [(lambda r=r: nv.mx_linear_w4a4(x, r[0], r[1], out=y, workspace=ws)) for r in rot]
    elif what == "kv_gather":
        kw = WL.KV_PREFILL
        table, lens, dst, nb, out_rows = kw.layout()
        td, ld, dd = (torch.from_numpy(a).cuda() for a in (table, lens, dst))
        codes, scales = kw.cache("nvfp4", nb)
        ts = torch.tensor([kw.KV_TSCALE], dtype=torch.float32, device="cuda")
        per_copy = codes.size + scales.size + 2 * out_rows * kw.heads * kw.head_dim
        items = [(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                  torch.empty((out_rows, kw.heads, kw.head_dim), dtype=torch.float16, device="cuda"))
                 for _ in range(copies_needed(per_copy))]
        calls = [(lambda c=c, s=s, o=o: nv.kv_gather(c, s, ts, td, ld, dd, o, fmt="nvfp4")) for (c, s, o) in items]
    elif what == "moe_prefill":
        pw = WL.MOE_PREFILL
        base = dev_bf16(pw.base_weight())
        stack = torch.stack([(base.float() * pw.expert_scale(i)).to(torch.bfloat16) for i in range(pw.experts)])
        packed, scales, tscale = nv.quantize_experts(stack)
        del stack, base
        route = torch.from_numpy(pw.random_routes()).cuda()
        x = dev_bf16(WL.activations(pw.t, pw.k))
        y = torch.empty((pw.t, pw.topk, pw.n), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(nv.linear_grouped_workspace_bytes(pw.t, pw.topk, pw.experts), dtype=torch.uint8,
                         device="cuda")
        calls = [lambda: nv.linear_grouped(x, route, packed, scales, tscale, out=y, workspace=ws)]
    elif what == "copy":
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        calls = [lambda: dst.copy_(src)]
    else:
        nv.lib()
        wl = WL.WORKLOADS["decode" if what == "decode" else "prefill"]
        m = {"decode": 1, "prefill": 512, "prefill2048": 2048}[what]
        packed, scales, tscale = nv.quantize(dev_bf16(wl.weight()))
        x = dev_bf16(wl.activations(m))
        rot = Rotated(packed, scales, tscale, copies_needed(packed.numel() + scales.numel()))
        y = torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda")
        calls = linear_calls(x, rot, y)
    torch.cuda.synchronize()
    if graph:
        g = graph_of(calls)
        warm_graph(g)
        for _ in range(-(-launches // len(calls))):
            g.replay()
    else:
        for i in range(launches):
            calls[i % len(calls)]()
    torch.cuda.synchronize()
    print(f"profile run done: {what} x{launches}{' (graph replays)' if graph else ''}", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3700)
    ap.add_argument("--warmup", type=int, default=370)
    ap.add_argument("--rows", default="all", help="'all' or 'none': also measure the other rows of the hot path")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--cpu-baseline-only", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--profile", choices=["decode", "prefill", "prefill2048", "copy", "moe_prefill", "kv_gather", "mx_w4a4",
                                              "nvfp4_w4a4", "quantize", "dequant", "linear", "prepared", "stream"], default=None,
                    help="short untimed run of one kernel for hardware-counter passes; prints no JSON")
    ap.add_argument("--launches", type=int, default=40, help="launches in a --profile run")
    ap.add_argument("--graph", action="store_true", help="--profile run: replay the rotated launches as one HIP graph")
    ap.add_argument("--workload", default="small_m_up", help="workload of a --profile linear run")
    ap.add_argument("--m", type=int, default=8, help="activation rows of a --profile linear run")
    args = ap.parse_args()
    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline_run(args.cpu_budget)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported. The library runs the linear on "
              f"one MI355X; a multi-GPU layer would shard the weight rows (N) or whole 16-element K blocks "
              f"across GPUs above this library.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.profile:
        profile_run(args.profile, args.launches, args.workload, args.m, args.graph)
        return
    torch.cuda.set_device(0)
    nv.lib()

    wl = WL.WORKLOADS["decode"]
    m, n, k = 1, wl.n, wl.k
    log(f"decode workload: quantizing {n}x{k}")
    w = wl.weight()
    packed, scales, tscale = nv.quantize(dev_bf16(w))
    x = dev_bf16(wl.activations(m))
    del w

    c = copies_needed(packed.numel() + scales.numel())
    rot = Rotated(packed, scales, tscale, c)
    yout = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    calls = linear_calls(x, rot, yout)
    full = graph_of(calls)
    rem = args.steps % c
    part = graph_of(calls[:rem]) if rem else None
    log(f"{c} rotated copies; warmup {args.warmup}, timed {args.steps} steps")
    for _ in range(max(1, args.warmup // c)):
        full.replay()
    torch.cuda.synchronize()
    warm_graph(full)   # the same 0.1 s of loaded clock as every row below
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps // c):
        full.replay()
    if part is not None:
        part.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = linear_bytes(m, n, k)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"decode GEMV: {ms * 1e3:.3f} us/call, {gbs:.1f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM peak); wall {wall:.2f} s")
    digest = source_digest(["gemv.hip", "device_common.hpp"])

    rows = {}
    if args.rows == "all":
        for wname, mm, reps in [("gate_up", 1, 30), ("small_m_down", 1, 30), ("small_m_up", 8, 30),
                                ("small_m_up", 32, 30), ("small_m_down", 8, 30), ("small_m_down", 32, 30),
                                ("prefill", 512, 10), ("prefill", 2048, 3),
                                ("prefill_down", 512, 10), ("prefill_down", 2048, 3)]:
            key = f"linear_{wname}_m{mm}"
            log(f"row {key}")
            rows[key] = bench_linear_row(wname, mm, reps)
            log(f"  {rows[key]}")
        for wname, mm, reps in [("small_m_up", 8, 30), ("small_m_up", 32, 30), ("small_m_down", 8, 30),
                                ("small_m_down", 32, 30), ("gate_up", 1, 30), ("decode", 1, 30),
                                ("small_m_down", 1, 30)]:
            key = f"prepared_{wname}_m{mm}"
            log(f"row {key}")
            rows[key] = bench_prepared_row(wname, mm, reps)
            log(f"  {rows[key]}")
        rows["prepare_small_m_up_17408x5120"] = bench_prepare_row(20)
        log(f"  prepare: {rows['prepare_small_m_up_17408x5120']}")
        log("rows streaming read")
        rows.update(bench_stream_rows(30))
        log(f"  {[(k, v['us_per_call'], v['gb_s']) for k, v in rows.items() if k.startswith('stream_read')]}")
        log("rows quantize/dequant")
        rows.update(bench_quant_rows(20))
        log(f"  {rows['quantize_decode_5120x5120']} {rows['dequant_decode_5120x5120']}")
        log("rows MoE")
        rows.update(bench_moe_rows(reps))
        log(f"  {rows['moe_routed_decode_top8']}")
        log(f"  {rows['moe_grouped_prefill_t2048_top8']}")
        log("rows KV gather")
        rows.update(bench_kv_rows(20))
        log(f"  {rows['kv_gather_nvfp4_f16']} {rows['kv_gather_mxfp4_f16']}")
        log("rows MXFP4 W4A4")
        rows.update(bench_mx_rows(10))
        log(f"  {rows['mx_w4a4_prefill_m512']} {rows['mx_w4a4_prefill_m2048']}")
        log("rows NVFP4 W4A4")
        for mm, reps_w in ((512, 10), (2048, 3)):
            rows.update(bench_w4a4_nvfp4_row(mm, reps_w))
        log(f"  {rows['nvfp4_w4a4_prefill_m512']} {rows['nvfp4_w4a4_prefill_m2048']}")

    # Every HBM-bound row also as a fraction of the measured streaming-read rate of the nearest size.
    streams = sorted((v["bytes"], v["gb_s"]) for k, v in rows.items() if k.startswith("stream_read"))
    if streams:
        for key, r in rows.items():
            if "gb_s" in r and "hbm_frac" in r and not key.startswith("stream_read"):
                nb = r.get("bytes") or linear_bytes(r.get("m", 1), r.get("n", 1), r.get("k", 1))
                ref = min(streams, key=lambda sv: abs(sv[0] - nb))[1]
                r["measured_read_gb_s"] = ref
                r["measured_read_frac"] = round(r["gb_s"] / ref, 4)
    head_read = min(streams, key=lambda sv: abs(sv[0] - linear_bytes(m, n, k)))[1] if streams else None
    log("cpu baseline (oracle)")
    cpu = cpu_baseline(args.cpu_budget)
    result = {
        "metric": "NVFP4 W4A16 linear: achieved HBM GB/s (M=1..32), TFLOP/s (M=512), % of peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded BF16 normals, RTN-quantized to NVFP4 on the GPU)",
        "config": {"workload": "decode GEMV: M=1, N=5120, K=5120, 1% outlier input columns x8",
                   "m": m, "n": n, "k": k, "rotated_weight_copies": c,
                   "timing": "HIP-graph replay of the rotated launch sequence, HIP events on the launch stream",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("gemv_decode_5120x5120", digest),
                     "kernel": "gemv_ks_kernel<3, 1>", "bytes_per_launch": nbytes,
                     "avg_launch_us": round(ms * 1e3, 3),
                     "measured_read_gb_s": head_read,
                     "measured_read_frac": round(gbs / head_read, 4) if head_read else None},
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
