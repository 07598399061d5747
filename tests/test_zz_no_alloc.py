"""ga_gelu_and_mul_sparse_noalloc (the entry point for callers that cannot
allocate device memory) against ga_gelu_and_mul_sparse_ws with a caller
workspace, both called through the C-ABI: two calls in a row on split-row
shapes, the second smaller, each bit-identical to the workspace entry point
(the same plan and kernels) and within tolerance of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import gated_activation_amd as ga
import oracle
import synth
from parity import BF16, Z95, bits_of, compare, decode, sentinel_buffer, to_device

pytestmark = pytest.mark.gpu
L = ga.lib


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("shapes", [((16, 32768, None), (4, 32768, 3)), ((64, 65536, None), (1, 65536, None))],
                         ids=["16x32768_then_4x32768_live3", "64x65536_then_1x65536"])
def test_noalloc_matches_workspace_entry_point(shapes):
    assert torch.cuda.is_available(), "this test needs a GPU"
    o = oracle.get()
    for T, d, live in shapes:
        print(f"noalloc T={T} d={d} live={live}", flush=True)
        assert T <= ga.GA_SPLIT_PLAN_ROWS
        xb = synth.gelu_large(T, d)
        x = to_device(xb, BF16)
        live_t = None if live is None else torch.tensor([live], dtype=torch.int32, device="cuda")
        live_p = None if live_t is None else _ptr(live_t)
        plan = ga.plan_gelu_and_mul_sparse(T, d, ga.GA_BF16)
        _, out_na = sentinel_buffer(T, d, BF16)
        _, out_ws = sentinel_buffer(T, d, BF16)
        ws = torch.zeros(L.ga_gelu_and_mul_sparse_workspace_bytes(T), dtype=torch.uint8, device="cuda")
        z = ctypes.c_float(Z95)
        st = L.ga_gelu_and_mul_sparse_noalloc(_ptr(x), _ptr(out_na), T, d, ga.GA_BF16, z, live_p, _stream())
        assert st == ga.GA_OK, L.ga_last_error()
        st = L.ga_gelu_and_mul_sparse_ws(_ptr(x), _ptr(out_ws), T, d, ga.GA_BF16, z, live_p, _ptr(ws),
                                         ws.numel(), _stream())
        assert st == ga.GA_OK, L.ga_last_error()
        torch.cuda.synchronize()
        a, b = bits_of(out_na, BF16), bits_of(out_ws, BF16)
        assert np.array_equal(a, b), f"T={T} d={d}: the two entry points differ (split plan {plan.splits})"
        n = T if live is None else min(max(live, 0), T)
        ref, stats = o.gelu_and_mul_sparse(xb[:n], BF16, Z95, want_stats=True)
        compare(a[:n], ref, BF16, gate=decode(xb[:n, :d], BF16), stats=stats, label=f"noalloc T{T} d{d}")
        assert np.all(a[n:] == synth.SENTINEL[BF16])
        assert plan.path == 0 and plan.splits > 1      # split rows: the scratch array is used
