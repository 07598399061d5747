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


def test_graph_replay_packed_unaligned_and_round_trip():
    """The packed-rows path (short rows, aligned and odd d), the unaligned
    path (odd d), the round-trip form and gelu_and_mul captured together,
    replayed under changing live counts and checked on every replay."""
    o = oracle.get()
    cases = []
    for T, d, rt in ((1000, 128, False), (700, 101, False), (300, 2047, False), (200, 4096, True)):
        xb = synth.gelu_offset_rows(T, d, seed=T + d)
        if rt:
            ref, st = o.gelu_and_mul_sparse_rt(xb, BF16, Z95)
        else:
            ref, st = o.gelu_and_mul_sparse(xb, BF16, Z95, want_stats=True)
        _, out = sentinel_buffer(T, d, BF16)
        live = torch.tensor([T], dtype=torch.int32, device="cuda")
        cases.append(dict(T=T, d=d, rt=rt, xb=xb, x=to_device(xb, BF16), ref=ref, st=st, out=out, live=live))
    assert ga.plan_gelu_and_mul_sparse(1000, 128, ga.GA_BF16).path == 3
    assert ga.plan_gelu_and_mul_sparse(700, 101, ga.GA_BF16).path == 3
    assert ga.plan_gelu_and_mul_sparse(300, 2047, ga.GA_BF16).path == 2
    xm_b = synth.gelu_iid(500, 1536, seed=31)
    ref_m = o.gelu_and_mul(xm_b, BF16, True)
    xm = to_device(xm_b, BF16)
    _, out_m = sentinel_buffer(500, 1536, BF16)
    live_m = torch.tensor([500], dtype=torch.int32, device="cuda")
    sentinel = int(synth.SENTINEL[BF16])

    def launch():
        for c in cases:
            ga.gelu_and_mul_sparse(c["x"], Z95, out=c["out"], live_rows=c["live"], round_intermediates=c["rt"])
        ga.gelu_and_mul(xm, "tanh", out=out_m, live_rows=live_m)

    launch()
    torch.cuda.synchronize()
    eager = [bits_of(c["out"], BF16).copy() for c in cases]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    torch.cuda.synchronize()
    for step, frac in enumerate((1.0, 0.0, 0.37, 1.5, 0.01)):
        for c in cases:
            c["out"].view(torch.int16).fill_(sentinel)
            c["live"].fill_(int(c["T"] * frac))
        out_m.view(torch.int16).fill_(sentinel)
        live_m.fill_(int(500 * frac))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for c, eg in zip(cases, eager):
            k = min(int(c["T"] * frac), c["T"])
            got = bits_of(c["out"], BF16)
            label = f"graph T{c['T']} d{c['d']} rt{c['rt']} step {step}"
            # every replay reproduces the eager launch bit for bit ...
            assert np.array_equal(got[:k], eg[:k]), label
            # ... which matches the oracle (the round-trip form within its
            # cutoff-candidate rule, checked in test_gpu_roundtrip.py)
            if not c["rt"]:
                gate = decode(c["xb"][:k, :c["d"]], BF16)
                compare(got[:k], c["ref"][:k], BF16, gate=gate, stats=c["st"][:, :k], label=label)
            assert np.all(got[k:] == synth.SENTINEL[BF16]), label
        km = min(int(500 * frac), 500)
        got_m = bits_of(out_m, BF16)
        compare(got_m[:km], ref_m[:km], BF16, label=f"graph gelu_and_mul step {step}")
        assert np.all(got_m[km:] == synth.SENTINEL[BF16])


def test_default_workspace_survives_capture_and_later_calls():
    """A few-row call captured with the binding's own workspace (no
    workspace= argument) takes the split path; an eager call of 2048 rows on
    the same stream afterwards must not replace or free that workspace, so
    every replay still finds it and matches the oracle (Megatron-LM PR 6328,
    What changed and why: the buffers a graph captures stay fixed while the
    per-step data changes)."""
    Tq, dq, Tb, db = 8, 32768, 2048, 16384
    o = oracle.get()
    xq_b = synth.gelu_large(Tq, dq)
    ref_q, st_q = o.gelu_and_mul_sparse(xq_b, BF16, Z95, want_stats=True)
    xb_b = synth.gelu_large(Tb, db)
    pq = ga.plan_gelu_and_mul_sparse(Tq, dq, ga.GA_BF16)
    assert pq.path == 0 and pq.splits > 1                 # split rows: the workspace is used
    assert ga.plan_gelu_and_mul_sparse(Tb, db, ga.GA_BF16).splits == 1
    s = torch.cuda.Stream()
    key = (torch.cuda.current_device(), s.cuda_stream)
    assert key not in ga.held_workspaces()       # a fresh stream: nothing reserved yet
    xq, xb = to_device(xq_b, BF16), to_device(xb_b, BF16)
    _, out_q = sentinel_buffer(Tq, dq, BF16)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        ga.gelu_and_mul_sparse(xq, Z95, out=out_q)
    torch.cuda.synchronize()
    # the captured call allocated the stream's workspace (inside the capture)
    captured_ptr = ga.held_workspaces()[key]
    # an eager call with many rows on the same stream, then eager few-row calls
    with torch.cuda.stream(s):
        out_b = ga.gelu_and_mul_sparse(xb, Z95)
        ga.gelu_and_mul_sparse(xq, Z95)
    torch.cuda.synchronize()
    assert ga.held_workspaces()[key] == captured_ptr
    ref_b, st_b = o.gelu_and_mul_sparse(xb_b[:64], BF16, Z95, want_stats=True)
    compare(bits_of(out_b[:64], BF16), ref_b, BF16, gate=decode(xb_b[:64, :db], BF16), stats=st_b,
            label="eager T2048 beside the graph")
    gate_q = decode(xq_b[:, :dq], BF16)
    sentinel = int(synth.SENTINEL[BF16])
    for step in range(4):
        out_q.view(torch.int16).fill_(sentinel)
        with torch.cuda.stream(s):
            ga.gelu_and_mul_sparse(xq, Z95)      # eager use of the workspace between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        compare(bits_of(out_q, BF16), ref_q, BF16, gate=gate_q, stats=st_q, label=f"captured split, replay {step}")
    assert ga.held_workspaces()[key] == captured_ptr


def test_reserved_workspace_is_the_one_a_capture_uses():
    """reserve_workspace(stream=s) before capture: the captured few-row call
    uses that workspace (zeroed outside the graph) and splits its rows."""
    Tq, dq = 4, 32768
    o = oracle.get()
    xq_b = synth.gelu_large(Tq, dq)
    ref_q, st_q = o.gelu_and_mul_sparse(xq_b, BF16, Z95, want_stats=True)
    pq = ga.plan_gelu_and_mul_sparse(Tq, dq, ga.GA_BF16)
    assert pq.path == 0 and pq.splits > 1
    s = torch.cuda.Stream()
    ws = ga.reserve_workspace(stream=s)
    assert ws.numel() == ga.WORKSPACE_BYTES
    key = (torch.cuda.current_device(), s.cuda_stream)
    assert ga.held_workspaces()[key] == ws.data_ptr()
    xq = to_device(xq_b, BF16)
    _, out_q = sentinel_buffer(Tq, dq, BF16)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        ga.gelu_and_mul_sparse(xq, Z95, out=out_q)
    torch.cuda.synchronize()
    assert ga.held_workspaces()[key] == ws.data_ptr()
    for step in range(3):
        out_q.view(torch.int16).fill_(int(synth.SENTINEL[BF16]))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        compare(bits_of(out_q, BF16), ref_q, BF16, gate=decode(xq_b[:, :dq], BF16), stats=st_q,
                label=f"reserved workspace, replay {step}")
