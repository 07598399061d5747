"""Both operations recorded once into a HIP graph and replayed while the
device-side live count changes (Megatron-LM PR 6328: the grid is baked in at
capture from the buffer bound, never from the per-step count; vLLM PR 48498
covers the op under CUDA Graph capture).  Each replay is checked against the
oracle, with the program's own eager work and a synchronisation in between."""
import numpy as np
import pytest
import torch

import gated_activation_amd as ga
import oracle
import synth
from parity import BF16, Z95, bits_of, compare, decode, sentinel_buffer, to_device

pytestmark = pytest.mark.gpu


def test_graph_replay_with_changing_live_counts():
    Ms, ds = 4096, 768
    Tg, dg = 256, 8192
    Tq, dq = 8, 32768        # few long rows: the split-row path
    xs_b = synth.moe_buffer(Ms, ds, seed=11)
    xg_b = synth.gelu_offset_rows(Tg, dg, seed=12)
    o = oracle.get()
    ref_s = o.silu_and_mul_bounded(xs_b, BF16, Ms)
    ref_g, st_g = o.gelu_and_mul_sparse(xg_b, BF16, Z95, want_stats=True)
    xq_b = synth.gelu_large(Tq, dq)
    ref_q, st_q = o.gelu_and_mul_sparse(xq_b, BF16, Z95, want_stats=True)
    assert ga.plan_gelu_and_mul_sparse(Tq, dq, ga.GA_BF16).splits > 1
    xs, xg, xq = to_device(xs_b, BF16), to_device(xg_b, BF16), to_device(xq_b, BF16)
    _, out_q = sentinel_buffer(Tq, dq, BF16)
    live_q = torch.tensor([Tq], dtype=torch.int32, device="cuda")
    ws_q = torch.zeros(ga.lib.ga_gelu_and_mul_sparse_workspace_bytes(Tq), dtype=torch.uint8, device="cuda")
    _, out_s = sentinel_buffer(Ms, ds, BF16)
    _, out_g = sentinel_buffer(Tg, dg, BF16)
    live_s = torch.tensor([Ms], dtype=torch.int32, device="cuda")
    live_g = torch.tensor([Tg], dtype=torch.int32, device="cuda")
    sentinel = int(synth.SENTINEL[BF16])  # 0x7FA5 fits int16

    # warm-up outside capture, then record
    ga.silu_and_mul_bounded(xs, live_s, out=out_s)
    ga.gelu_and_mul_sparse(xg, Z95, out=out_g, live_rows=live_g)
    ga.gelu_and_mul_sparse(xq, Z95, out=out_q, live_rows=live_q, workspace=ws_q)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ga.silu_and_mul_bounded(xs, live_s, out=out_s)
        ga.gelu_and_mul_sparse(xg, Z95, out=out_g, live_rows=live_g)
        ga.gelu_and_mul_sparse(xq, Z95, out=out_q, live_rows=live_q, workspace=ws_q)
    torch.cuda.synchronize()

    gate = decode(xg_b[:, :dg], BF16)
    gate_q = decode(xq_b[:, :dq], BF16)
    for n_s, n_g in ((64, 1), (4096, 256), (0, 0), (1000, 77), (5000, 300), (17, 128)):
        n_q = n_g % (Tq + 1)
        out_s.view(torch.int16).fill_(sentinel)
        out_g.view(torch.int16).fill_(sentinel)
        out_q.view(torch.int16).fill_(sentinel)
        live_s.fill_(n_s)
        live_g.fill_(n_g)
        live_q.fill_(n_q)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ks, kg = min(max(n_s, 0), Ms), min(max(n_g, 0), Tg)
        got_s, got_g = bits_of(out_s, BF16), bits_of(out_g, BF16)
        compare(got_s[:ks], ref_s[:ks], BF16, label=f"graph silu {n_s}")
        assert np.all(got_s[ks:] == synth.SENTINEL[BF16])
        compare(got_g[:kg], ref_g[:kg], BF16, gate=gate[:kg], stats=st_g[:, :kg], label=f"graph gelu {n_g}")
        assert np.all(got_g[kg:] == synth.SENTINEL[BF16])
        got_q = bits_of(out_q, BF16)
        compare(got_q[:n_q], ref_q[:n_q], BF16, gate=gate_q[:n_q], stats=st_q[:, :n_q], label=f"graph split {n_q}")
        assert np.all(got_q[n_q:] == synth.SENTINEL[BF16])
