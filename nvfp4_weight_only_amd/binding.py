"""Thin ctypes binding of libnvfp4.so (argument marshalling only).

Every computation runs in the library's HIP kernels.  torch provides device
memory and the current HIP stream; there is no CPU or PyTorch fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple, Union

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4.so")
_lib: Optional[ctypes.CDLL] = None

KERNEL_AUTO, KERNEL_GEMV, KERNEL_SMALL_M, KERNEL_PREFILL = 0, 1, 2, 3
KERNEL_IDS = {"auto": KERNEL_AUTO, "gemv": KERNEL_GEMV, "small_m": KERNEL_SMALL_M, "prefill": KERNEL_PREFILL}

# Status codes (include/nvfp4.h).
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_UNSUPPORTED, ERR_ALIAS = range(7)

# Every symbol include/nvfp4.h declares.
EXPORTED = ("nvfp4_status_string", "nvfp4_version", "nvfp4_quantize", "nvfp4_amax_accumulate",
            "nvfp4_quantize_with_amax", "nvfp4_dequant", "nvfp4_linear", "nvfp4_linear_forced",
            "nvfp4_linear_ws", "nvfp4_quantize_experts", "nvfp4_dequant_experts", "nvfp4_linear_routed",
            "nvfp4_linear_grouped", "nvfp4_kv_gather", "nvfp4_mx_quantize", "nvfp4_mx_dequant", "nvfp4_mx_gemm",
            "nvfp4_mx_linear_w4a4", "nvfp4_linear_workspace_bytes", "nvfp4_linear_grouped_workspace_bytes",
            "nvfp4_mx_linear_w4a4_workspace_bytes", "nvfp4_linear_w4a4", "nvfp4_linear_w4a4_workspace_bytes",
            "nvfp4_linear_noalloc", "nvfp4_linear_noalloc_max_bytes", "nvfp4_prepared_bytes", "nvfp4_prepare",
            "nvfp4_dequant_prepared", "nvfp4_linear_prepared_workspace_bytes", "nvfp4_linear_prepared",
            "nvfp4_stream_read", "nvfp4_stream_read_sink_words", "nvfp4_quantize_ws",
            "nvfp4_quantize_workspace_bytes")


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().nvfp4_status_string(status).decode()}")


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libnvfp4.so (built in-tree by nvfp4_weight_only_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m nvfp4_weight_only_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.nvfp4_status_string.argtypes = [i32]
        L.nvfp4_status_string.restype = ctypes.c_char_p
        L.nvfp4_version.argtypes = []
        L.nvfp4_version.restype = ctypes.c_char_p
        L.nvfp4_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp]
        L.nvfp4_quantize_ws.argtypes = [vp, i64, i64, vp, vp, vp, vp, i64, vp]
        L.nvfp4_quantize_workspace_bytes.argtypes = []
        L.nvfp4_amax_accumulate.argtypes = [vp, i64, i64, vp, vp]
        L.nvfp4_quantize_with_amax.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
        L.nvfp4_dequant.argtypes = [vp, vp, vp, i64, i64, vp, vp]
        L.nvfp4_linear.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.nvfp4_linear_forced.argtypes = [i32, vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.nvfp4_linear_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.nvfp4_linear_noalloc_max_bytes.argtypes = []
        L.nvfp4_linear_noalloc_max_bytes.restype = i64
        L.nvfp4_prepared_bytes.argtypes = [i64, i64]
        L.nvfp4_prepare.argtypes = [vp, vp, i64, i64, vp, vp]
        L.nvfp4_dequant_prepared.argtypes = [vp, vp, i64, i64, vp, vp]
        L.nvfp4_linear_prepared_workspace_bytes.argtypes = [i64, i64, i64]
        L.nvfp4_linear_prepared.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, i64, vp]
        L.nvfp4_stream_read.argtypes = [vp, i64, vp, vp]
        L.nvfp4_stream_read_sink_words.argtypes = [i64]
        L.nvfp4_linear_ws.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
        L.nvfp4_quantize_experts.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
        L.nvfp4_dequant_experts.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp]
        L.nvfp4_linear_routed.argtypes = [vp, i64, i64, vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.nvfp4_linear_grouped.argtypes = [vp, i64, i64, vp, i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
        L.nvfp4_kv_gather.argtypes = [i32, i32, vp, vp, vp, i64, i64, i64, i64, vp, i64, vp, vp, i64, vp, i64, vp]
        L.nvfp4_mx_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        L.nvfp4_mx_dequant.argtypes = [vp, vp, i64, i64, vp, vp]
        L.nvfp4_mx_gemm.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, vp]
        L.nvfp4_mx_linear_w4a4.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, i64, vp]
        L.nvfp4_mx_linear_w4a4_workspace_bytes.argtypes = [i64, i64]
        L.nvfp4_linear_w4a4.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
        L.nvfp4_linear_w4a4_workspace_bytes.argtypes = [i64, i64]
        L.nvfp4_linear_workspace_bytes.argtypes = [i64, i64, i64]
        L.nvfp4_linear_grouped_workspace_bytes.argtypes = [i64, i64, i64]
        for name in EXPORTED[2:]:
            getattr(L, name).restype = i64 if name.endswith(("_workspace_bytes", "_max_bytes", "_prepared_bytes", "_sink_words")) \
                else i32
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != OK:
        raise NVFP4Error(status, what)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize(w: torch.Tensor, workspace: Union[str, None, torch.Tensor] = "auto"
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """BF16 [n, k] -> (packed uint8 [n, k/2], scales uint8 [n, k/16], tscale float32 [1]).

    workspace: "auto" runs nvfp4_quantize_ws (two launches) on the binding-owned workspace of the current
    device and stream; None runs nvfp4_quantize (three launches); a uint8 device tensor is passed through.
    The outputs are the same bits either way."""
    _need(w, torch.bfloat16, "w")
    n, k = w.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // 16), dtype=torch.uint8, device=w.device)
    tscale = torch.empty((1,), dtype=torch.float32, device=w.device)
    stream = _stream(w)
    head = (w.data_ptr(), n, k, packed.data_ptr(), scales.data_ptr(), tscale.data_ptr())
    if workspace is None:
        _check(lib().nvfp4_quantize(*head, stream), "nvfp4_quantize")
        return packed, scales, tscale
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
        ws = _workspace_for(w.device, stream, lib().nvfp4_quantize_workspace_bytes(), kind="quantize")
    else:
        _need(workspace, torch.uint8, "workspace")
        ws = workspace
    _check(lib().nvfp4_quantize_ws(*head, ws.data_ptr(), ws.numel(), stream), "nvfp4_quantize_ws")
    return packed, scales, tscale


def amax_accumulate(w: torch.Tensor, amax: torch.Tensor) -> None:
    """amax <- max(amax, max|w|) on the device (amax: float32 [1], caller-initialised)."""
    _need(w, torch.bfloat16, "w")
    _need(amax, torch.float32, "amax")
    n, k = w.shape
    _check(lib().nvfp4_amax_accumulate(w.data_ptr(), n, k, amax.data_ptr(), _stream(w)), "nvfp4_amax_accumulate")


def quantize_with_amax(w: torch.Tensor, amax: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Quantize one member of a merged linear against a shared amax (see nvfp4_quantize_with_amax)."""
    _need(w, torch.bfloat16, "w")
    _need(amax, torch.float32, "amax")
    n, k = w.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // 16), dtype=torch.uint8, device=w.device)
    tscale = torch.empty((1,), dtype=torch.float32, device=w.device)
    _check(lib().nvfp4_quantize_with_amax(w.data_ptr(), n, k, amax.data_ptr(), packed.data_ptr(), scales.data_ptr(),
                                          tscale.data_ptr(), _stream(w)), "nvfp4_quantize_with_amax")
    return packed, scales, tscale


def quantize_shared(members) -> Tuple[list, torch.Tensor]:
    """Quantize the members of a merged linear (q/k/v, gate/up) against one tensor scale."""
    amax = torch.zeros((1,), dtype=torch.float32, device=members[0].device)
    for w in members:
        amax_accumulate(w, amax)
    outs = [quantize_with_amax(w, amax) for w in members]
    return [(p, s) for p, s, _ in outs], outs[0][2]


def dequant(packed: torch.Tensor, scales: torch.Tensor, tscale: torch.Tensor,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """NVFP4 -> BF16 [n, k] (into `out` when given)."""
    _need(packed, torch.uint8, "packed")
    _need(scales, torch.uint8, "scales")
    _need(tscale, torch.float32, "tscale")
    n, kh = packed.shape
    k = 2 * kh
    if scales.shape != (n, k // 16):
        raise ValueError("scales must be [n, k/16]")
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=packed.device)
    else:
        _need(out, torch.bfloat16, "out")
        if out.shape != (n, k):
            raise ValueError("out must be [n, k]")
    _check(lib().nvfp4_dequant(packed.data_ptr(), scales.data_ptr(), tscale.data_ptr(), n, k, out.data_ptr(),
                               _stream(packed)), "nvfp4_dequant")
    return out


def linear_workspace_bytes(m: int, n: int, k: int) -> int:
    """Workspace bytes nvfp4_linear_ws can use for this shape (0: none)."""
    b = lib().nvfp4_linear_workspace_bytes(m, n, k)
    if b < 0:
        raise ValueError(f"invalid linear shape m={m} n={n} k={k}")
    return b


# Workspaces owned by the binding, one per (device, stream): zero-filled when
# allocated, and left with zero counters by every call, so they are reused as is.
# A workspace that a larger shape supersedes is kept alive, never freed: a HIP
# graph captured earlier may still hold its address, and if the allocator handed
# that memory to another tensor, replays would write partial sums into it and
# start from counters that are not zero.
_workspaces: Dict[Tuple[int, int, str], torch.Tensor] = {}
_superseded: list = []


def _workspace_for(device: torch.device, stream: int, nbytes: int, kind: str = "split") -> torch.Tensor:
    """The binding-owned workspace of one (device, stream) for one kind of call.  "split": the split-K
    workspaces of the linear entry points, whose arrival counters every call leaves at zero; "quantize":
    nvfp4_quantize_ws's partial maxima (any contents), kept apart so that they never land on the counters."""
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream, kind)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            # The zero fill would only be recorded in the graph, not run, and the graph would own memory the
            # binding cannot keep zeroed: the workspace must exist before capture.
            raise RuntimeError(
                f"nvfp4: no workspace of {nbytes} bytes for this stream during graph capture: call linear() with "
                f"this shape once before capturing, or pass workspace= (a zero-filled uint8 device tensor)")
        # 256-byte aligned by the caching allocator; grown geometrically.
        size = max(nbytes, 2 * ws.numel() if ws is not None else 0)
        if ws is not None:
            _superseded.append(ws)
        ws = torch.zeros(size, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def linear(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, tscale: torch.Tensor,
           kernel: str = "auto", out: Optional[torch.Tensor] = None,
           workspace: Union[str, None, torch.Tensor] = "auto") -> torch.Tensor:
    """Y[m, n] = X[m, k] . W_hat[n, k]^T in BF16 (FP32 accumulation).

    kernel: "auto" (by m), or "gemv" / "small_m" / "prefill" to force one kernel (no workspace).
    workspace (auto kernel only): "auto" uses a binding-owned workspace for the current
    device and stream (nvfp4_linear_ws); None calls nvfp4_linear (no workspace); a uint8
    device tensor is passed through as the caller's workspace (zero-filled before first use).
    """
    _need(x, torch.bfloat16, "x")
    _need(packed, torch.uint8, "packed")
    _need(scales, torch.uint8, "scales")
    _need(tscale, torch.float32, "tscale")
    m, k = x.shape
    n = packed.shape[0]
    if packed.shape != (n, k // 2) or scales.shape != (n, k // 16):
        raise ValueError("packed/scales do not match x's k")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if out.shape != (m, n):
            raise ValueError("out must be [m, n]")
    kid = KERNEL_IDS[kernel]
    stream = _stream(x)
    head = (x.data_ptr(), m, n, k, packed.data_ptr(), scales.data_ptr(), tscale.data_ptr(), out.data_ptr())
    if kid != KERNEL_AUTO:
        _check(lib().nvfp4_linear_forced(kid, *head, stream), "nvfp4_linear_forced")
    elif workspace is None:
        _check(lib().nvfp4_linear(*head, stream), "nvfp4_linear")
    else:
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
            need = linear_workspace_bytes(m, n, k)
            ws = _workspace_for(x.device, stream, need) if need > 0 else None
        else:
            _need(workspace, torch.uint8, "workspace")
            ws = workspace
        wptr, wbytes = (ws.data_ptr(), ws.numel()) if ws is not None else (None, 0)
        _check(lib().nvfp4_linear_ws(*head, wptr, wbytes, stream), "nvfp4_linear_ws")
    return out


def linear_noalloc(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, tscale: torch.Tensor,
                   out: torch.Tensor) -> torch.Tensor:
    """The linear through nvfp4_linear_noalloc: the split-K workspace is the library's own device array, so the
    call allocates nothing (`out` is required for the same reason)."""
    _need(x, torch.bfloat16, "x")
    _need(packed, torch.uint8, "packed")
    _need(scales, torch.uint8, "scales")
    _need(tscale, torch.float32, "tscale")
    _need(out, torch.bfloat16, "out")
    m, k = x.shape
    n = packed.shape[0]
    if packed.shape != (n, k // 2) or scales.shape != (n, k // 16) or out.shape != (m, n):
        raise ValueError("packed/scales/out do not match x")
    _check(lib().nvfp4_linear_noalloc(x.data_ptr(), m, n, k, packed.data_ptr(), scales.data_ptr(),
                                      tscale.data_ptr(), out.data_ptr(), _stream(x)), "nvfp4_linear_noalloc")
    return out


def prepared_bytes(n: int, k: int) -> int:
    b = lib().nvfp4_prepared_bytes(n, k)
    if b < 0:
        raise ValueError(f"no kernel-native layout for n={n} k={k} (k must be a positive multiple of 128)")
    return b


def prepare(packed: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """Checkpoint layout (packed [n, k/2], scales [n, k/16]) -> the kernel-native layout (uint8, flat)."""
    _need(packed, torch.uint8, "packed")
    _need(scales, torch.uint8, "scales")
    n, kh = packed.shape
    k = 2 * kh
    if scales.shape != (n, k // 16):
        raise ValueError("scales must be [n, k/16]")
    out = torch.empty(prepared_bytes(n, k), dtype=torch.uint8, device=packed.device)
    _check(lib().nvfp4_prepare(packed.data_ptr(), scales.data_ptr(), n, k, out.data_ptr(), _stream(packed)),
           "nvfp4_prepare")
    return out


def dequant_prepared(prepared: torch.Tensor, tscale: torch.Tensor, n: int, k: int) -> torch.Tensor:
    """Kernel-native layout -> BF16 [n, k]."""
    _need(prepared, torch.uint8, "prepared")
    _need(tscale, torch.float32, "tscale")
    if prepared.numel() != prepared_bytes(n, k):
        raise ValueError("prepared does not match n, k")
    out = torch.empty((n, k), dtype=torch.bfloat16, device=prepared.device)
    _check(lib().nvfp4_dequant_prepared(prepared.data_ptr(), tscale.data_ptr(), n, k, out.data_ptr(),
                                        _stream(prepared)), "nvfp4_dequant_prepared")
    return out


def linear_prepared(x: torch.Tensor, prepared: torch.Tensor, tscale: torch.Tensor, n: int,
                    out: Optional[torch.Tensor] = None,
                    workspace: Union[str, None, torch.Tensor] = "auto") -> torch.Tensor:
    """Y[m, n] = X[m, k] . W_hat^T from the kernel-native layout (1 <= m <= 32).  workspace as for linear()."""
    _need(x, torch.bfloat16, "x")
    _need(prepared, torch.uint8, "prepared")
    _need(tscale, torch.float32, "tscale")
    m, k = x.shape
    if prepared.numel() != prepared_bytes(n, k):
        raise ValueError("prepared does not match n and x's k")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if out.shape != (m, n):
            raise ValueError("out must be [m, n]")
    stream = _stream(x)
    need = lib().nvfp4_linear_prepared_workspace_bytes(m, n, k)
    if need < 0:
        raise ValueError(f"invalid shape m={m} n={n} k={k}")
    if workspace is None or need == 0:
        ws = None
    elif isinstance(workspace, torch.Tensor):
        _need(workspace, torch.uint8, "workspace")
        ws = workspace
    else:
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
        ws = _workspace_for(x.device, stream, need)
    wptr, wbytes = (ws.data_ptr(), ws.numel()) if ws is not None else (None, 0)
    _check(lib().nvfp4_linear_prepared(x.data_ptr(), m, n, k, prepared.data_ptr(), tscale.data_ptr(),
                                       out.data_ptr(), wptr, wbytes, stream), "nvfp4_linear_prepared")
    return out


# ---------------------------------------------------------------------------
# Expert stacks (mixture-of-experts layers).
# ---------------------------------------------------------------------------
def quantize_experts(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """BF16 [e, n, k] -> (packed uint8 [e, n, k/2], scales uint8 [e, n, k/16], tscale float32 [e]).

    Matrix i equals quantize(w[i]) bit for bit (one tensor scale per expert).
    """
    _need(w, torch.bfloat16, "w")
    e, n, k = w.shape
    packed = torch.empty((e, n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((e, n, k // 16), dtype=torch.uint8, device=w.device)
    tscale = torch.empty((e,), dtype=torch.float32, device=w.device)
    _check(lib().nvfp4_quantize_experts(w.data_ptr(), e, n, k, packed.data_ptr(), scales.data_ptr(),
                                        tscale.data_ptr(), _stream(w)), "nvfp4_quantize_experts")
    return packed, scales, tscale


def _stack_shape(packed: torch.Tensor, scales: torch.Tensor, tscale: torch.Tensor):
    _need(packed, torch.uint8, "packed")
    _need(scales, torch.uint8, "scales")
    _need(tscale, torch.float32, "tscale")
    e, n, kh = packed.shape
    k = 2 * kh
    if scales.shape != (e, n, k // 16) or tscale.shape != (e,):
        raise ValueError("scales must be [e, n, k/16] and tscale [e]")
    return e, n, k


def dequant_experts(packed: torch.Tensor, scales: torch.Tensor, tscale: torch.Tensor) -> torch.Tensor:
    """NVFP4 expert stack -> BF16 [e, n, k]."""
    e, n, k = _stack_shape(packed, scales, tscale)
    out = torch.empty((e, n, k), dtype=torch.bfloat16, device=packed.device)
    _check(lib().nvfp4_dequant_experts(packed.data_ptr(), scales.data_ptr(), tscale.data_ptr(), e, n, k,
                                       out.data_ptr(), _stream(packed)), "nvfp4_dequant_experts")
    return out


def linear_routed(x: torch.Tensor, route: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                  tscale: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y[t, j, :] = X[t, :] . W_hat[route[t, j]]^T for an expert stack (top-k routed decode).

    x BF16 [t, k]; route int32 [t, topk] (device); packed/scales/tscale an expert stack.
    Expert ids outside [0, e) give zero rows.
    """
    _need(x, torch.bfloat16, "x")
    _need(route, torch.int32, "route")
    e, n, k = _stack_shape(packed, scales, tscale)
    t, kx = x.shape
    if kx != k:
        raise ValueError("x's k does not match the stack")
    if route.dim() != 2 or route.shape[0] != t:
        raise ValueError("route must be [t, topk]")
    topk = route.shape[1]
    if out is None:
        out = torch.empty((t, topk, n), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if out.shape != (t, topk, n):
            raise ValueError("out must be [t, topk, n]")
    _check(lib().nvfp4_linear_routed(x.data_ptr(), t, topk, route.data_ptr(), e, n, k, packed.data_ptr(),
                                     scales.data_ptr(), tscale.data_ptr(), out.data_ptr(), _stream(x)),
           "nvfp4_linear_routed")
    return out


def linear_grouped_workspace_bytes(t: int, topk: int, e: int) -> int:
    """Workspace bytes nvfp4_linear_grouped needs for t tokens, top-k routing over e experts."""
    b = lib().nvfp4_linear_grouped_workspace_bytes(t, topk, e)
    if b < 0:
        raise ValueError(f"invalid grouped shape t={t} topk={topk} e={e}")
    return b


def linear_grouped(x: torch.Tensor, route: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                   tscale: torch.Tensor, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Same result as linear_routed through the grouped GEMM (the prefill form).

    workspace: optional uint8 device tensor of at least linear_grouped_workspace_bytes(t, topk, e)
    bytes; one is allocated when it is not given.
    """
    _need(x, torch.bfloat16, "x")
    _need(route, torch.int32, "route")
    e, n, k = _stack_shape(packed, scales, tscale)
    t, kx = x.shape
    if kx != k:
        raise ValueError("x's k does not match the stack")
    if route.dim() != 2 or route.shape[0] != t:
        raise ValueError("route must be [t, topk]")
    topk = route.shape[1]
    if out is None:
        out = torch.empty((t, topk, n), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if out.shape != (t, topk, n):
            raise ValueError("out must be [t, topk, n]")
    need = linear_grouped_workspace_bytes(t, topk, e)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    else:
        _need(workspace, torch.uint8, "workspace")
    _check(lib().nvfp4_linear_grouped(x.data_ptr(), t, topk, route.data_ptr(), e, n, k, packed.data_ptr(),
                                      scales.data_ptr(), tscale.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                      workspace.numel(), _stream(x)),
           "nvfp4_linear_grouped")
    return out


# KV-cache formats and output types (include/nvfp4.h).
KV_FORMATS = {"nvfp4": 0, "mxfp4": 1}
_KV_GROUP = {"nvfp4": 16, "mxfp4": 32}


def kv_gather(codes: torch.Tensor, scales: torch.Tensor, tscale: Optional[torch.Tensor], block_table: torch.Tensor,
              seq_lens: torch.Tensor, dst_start: torch.Tensor, out: torch.Tensor, fmt: str = "nvfp4") -> torch.Tensor:
    """Gather a paged FP4 KV cache into `out` (FP16 or BF16 [out_rows, heads, head_dim]) in place.

    codes uint8 [num_blocks, block_size, heads, head_dim/2]; scales uint8 [num_blocks, block_size, heads,
    head_dim/G] (G = 16 for "nvfp4", with the FP32 tensor scale `tscale` [1]; G = 32 for "mxfp4", tscale None);
    block_table int32 [seqs, max_blocks], seq_lens and dst_start int32 [seqs], all on the device.
    """
    if fmt not in KV_FORMATS:
        raise ValueError(f"unknown KV format {fmt!r}")
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    for t, name in ((block_table, "block_table"), (seq_lens, "seq_lens"), (dst_start, "dst_start")):
        _need(t, torch.int32, name)
    if fmt == "nvfp4":
        _need(tscale, torch.float32, "tscale")
    if out.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("out must be float16 or bfloat16")
    _need(out, out.dtype, "out")
    if codes.dim() != 4 or scales.dim() != 4:
        raise ValueError("codes and scales must be [num_blocks, block_size, heads, *]")
    nb, bs, heads, half = codes.shape
    hd = 2 * half
    if tuple(scales.shape) != (nb, bs, heads, hd // _KV_GROUP[fmt]):
        raise ValueError("scales do not match codes")
    if out.dim() != 3 or out.shape[1] != heads or out.shape[2] != hd:
        raise ValueError("out must be [out_rows, heads, head_dim]")
    if block_table.dim() != 2 or seq_lens.shape != (block_table.shape[0],) or dst_start.shape != seq_lens.shape:
        raise ValueError("block_table must be [seqs, max_blocks], seq_lens and dst_start [seqs]")
    _check(lib().nvfp4_kv_gather(KV_FORMATS[fmt], 1 if out.dtype == torch.bfloat16 else 0, codes.data_ptr(),
                                 scales.data_ptr(), tscale.data_ptr() if tscale is not None else None, nb, bs, heads,
                                 hd, block_table.data_ptr(), block_table.shape[1], seq_lens.data_ptr(),
                                 dst_start.data_ptr(), block_table.shape[0], out.data_ptr(), out.shape[0],
                                 _stream(out)), "nvfp4_kv_gather")
    return out


def mx_quantize(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """BF16 [rows, k] -> MXFP4 (packed uint8 [rows, k/2], UE8M0 scales uint8 [rows, k/32])."""
    _need(w, torch.bfloat16, "w")
    rows, k = w.shape
    packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((rows, k // 32), dtype=torch.uint8, device=w.device)
    _check(lib().nvfp4_mx_quantize(w.data_ptr(), rows, k, packed.data_ptr(), scales.data_ptr(), _stream(w)),
           "nvfp4_mx_quantize")
    return packed, scales


def mx_dequant(packed: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """MXFP4 -> BF16 [rows, k]."""
    _need(packed, torch.uint8, "packed")
    _need(scales, torch.uint8, "scales")
    rows, k = packed.shape[0], packed.shape[1] * 2
    if tuple(scales.shape) != (rows, k // 32):
        raise ValueError("scales do not match packed")
    out = torch.empty((rows, k), dtype=torch.bfloat16, device=packed.device)
    _check(lib().nvfp4_mx_dequant(packed.data_ptr(), scales.data_ptr(), rows, k, out.data_ptr(), _stream(packed)),
           "nvfp4_mx_dequant")
    return out


def mx_gemm(xq: torch.Tensor, xs: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y [m, n] BF16 = Xq . Wq^T from MXFP4 operands (FP4 matrix cores)."""
    for t, name in ((xq, "xq"), (xs, "xs"), (wq, "wq"), (ws, "ws")):
        _need(t, torch.uint8, name)
    m, k = xq.shape[0], xq.shape[1] * 2
    n = wq.shape[0]
    if wq.shape[1] * 2 != k or tuple(xs.shape) != (m, k // 32) or tuple(ws.shape) != (n, k // 32):
        raise ValueError("operand shapes do not match")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=xq.device)
    _check(lib().nvfp4_mx_gemm(xq.data_ptr(), xs.data_ptr(), m, wq.data_ptr(), ws.data_ptr(), n, k, out.data_ptr(),
                               _stream(xq)), "nvfp4_mx_gemm")
    return out


def mx_linear_w4a4(x: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y [m, n] BF16 = MXFP4(X) . Wq^T: X quantized to MXFP4 on the stream, then the FP4 GEMM."""
    _need(x, torch.bfloat16, "x")
    _need(wq, torch.uint8, "wq")
    _need(ws, torch.uint8, "ws")
    m, k = x.shape
    n = wq.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    need = lib().nvfp4_mx_linear_w4a4_workspace_bytes(m, k)
    if need < 0:
        raise ValueError(f"invalid shape m={m} k={k}")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_mx_linear_w4a4(x.data_ptr(), m, n, k, wq.data_ptr(), ws.data_ptr(), out.data_ptr(),
                                      workspace.data_ptr(), workspace.numel(), _stream(x)), "nvfp4_mx_linear_w4a4")
    return out


def linear_w4a4_workspace_bytes(m: int, k: int) -> int:
    return int(lib().nvfp4_linear_w4a4_workspace_bytes(m, k))


def linear_w4a4(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, tscale: torch.Tensor,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y [m, n] BF16 = NVFP4(X) . W_hat^T: X quantized to NVFP4 on the stream (its own tensor scale)."""
    _need(x, torch.bfloat16, "x")
    _need(packed, torch.uint8, "packed")
    _need(scales, torch.uint8, "scales")
    _need(tscale, torch.float32, "tscale")
    m, k = x.shape
    n = packed.shape[0]
    if packed.shape != (n, k // 2) or scales.shape != (n, k // 16):
        raise ValueError("packed/scales do not match x's k")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, "out")
        if out.shape != (m, n):
            raise ValueError("out must be [m, n]")
    need = linear_w4a4_workspace_bytes(m, k)
    if need < 0:
        raise ValueError(f"invalid shape m={m} k={k}")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_linear_w4a4(x.data_ptr(), m, n, k, packed.data_ptr(), scales.data_ptr(), tscale.data_ptr(),
                                   out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(x)),
           "nvfp4_linear_w4a4")
    return out
