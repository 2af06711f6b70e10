"""GPU test of nvfp4_linear_noalloc (the linear whose split-K workspace is the
library's own device array): called through the C ABI, its output must equal
nvfp4_linear_ws's with a caller workspace bit for bit, and the oracle's within
the linear's tolerance, on consecutive calls of different sizes."""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from nvfp4_weight_only_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _case(nv, m, n, k, seed):
    w = WL.normal_bf16((n, k), 0.02, seed)
    x = WL.normal_bf16((m, k), 1.0, seed + 1)
    packed, scales, tscale = nv.quantize(_dev_bf16(w))
    rp, rs, rt = O.quantize(w)
    assert np.array_equal(packed.cpu().numpy(), rp) and np.array_equal(scales.cpu().numpy(), rs)
    return _dev_bf16(x), (packed, scales, tscale), O.linear_ref(x, rp, rs, rt)


def test_linear_noalloc_matches_linear_ws():
    assert torch.cuda.is_available()
    import nvfp4_weight_only_amd as nv
    L = nv.lib()
    # Large split first, then a smaller one, then the first again: the shared array keeps the last call's
    # contents, and each call must still start from zero counters.
    shapes = [(32, 5120, 4096, 7000), (8, 300, 2048, 7010), (32, 5120, 4096, 7000), (1, 272, 1024, 7020)]
    for m, n, k, seed in shapes:
        x, (p, s, t), (y_ref, bound) = _case(nv, m, n, k, seed)
        need = L.nvfp4_linear_workspace_bytes(m, n, k)
        assert 0 <= need <= L.nvfp4_linear_noalloc_max_bytes()
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        st = L.nvfp4_linear_noalloc(x.data_ptr(), m, n, k, p.data_ptr(), s.data_ptr(), t.data_ptr(), y.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
        assert st == 0, L.nvfp4_status_string(st)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
        y_ws = torch.empty_like(y)
        st = L.nvfp4_linear_ws(x.data_ptr(), m, n, k, p.data_ptr(), s.data_ptr(), t.data_ptr(), y_ws.data_ptr(),
                               ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
        assert st == 0, L.nvfp4_status_string(st)
        torch.cuda.synchronize()
        got = _host_bits(y)
        assert np.array_equal(got, _host_bits(y_ws)), f"m={m} n={n} k={k}: differs from nvfp4_linear_ws"
        bad = O.linear_violations(WL.f32_from_bf16_bits(got).astype(np.float64), y_ref, bound)
        assert not bad.any(), f"m={m} n={n} k={k}: {int(bad.sum())} outputs outside the tolerance"
