"""Seeded random cases of gelu_and_mul_sparse on the GPU against the fp64
oracle (needs an MI355X).

Each case draws an element type, a row size (short, medium or long rows;
whole 16-byte vectors half of the time), a row count, input and output views
shifted off 16-byte alignment now and then, a live-row count or none, z, the
gate's scale and row mix (i.i.d. or with per-row offsets), and whether a
split-row workspace is passed.  The library plans every call itself, so the
cases land on whichever path it picks: one workgroup per row, packed short
rows, the unaligned and per-element paths, and few long rows split over
workgroups.  Live rows must match the oracle (the comparator's tolerance and
cutoff band); every element outside them, and around the output view, keeps
its sentinel bits; NaN around the input view must not reach the output.
"""
import numpy as np
import pytest
import torch

import gated_activation_amd as ga
import oracle
import synth
from parity import BF16, F16, F32, TORCH_DTYPE, Z95, Z99, bits_of, compare, decode, sentinel_buffer, to_device

pytestmark = pytest.mark.gpu

N_CASES = 400
MAX_ELEMS = 1_000_000  # T * d per case: the oracle stays within milliseconds


def draw(i):
    rng = np.random.default_rng(7919 * (i + 1))
    dt = (BF16, F16, F32)[rng.integers(3)]
    band = rng.integers(3)
    d = int(rng.integers(1, 300) if band == 0 else rng.integers(300, 9000) if band == 1
            else rng.integers(9000, 40000))
    if rng.random() < 0.5:
        d = max(8, d // 8 * 8)
    T = int(np.exp(rng.uniform(0.0, np.log(3000.0))))
    T = max(1, min(T, MAX_ELEMS // d))
    shifted = rng.random() < 0.3
    in_shift = int(rng.integers(0, 4)) if shifted else 0
    out_shift = int(rng.integers(0, 4)) if shifted else 0
    live = None if rng.random() < 0.5 else int(rng.integers(0, T + 3))
    z = float((0.0, Z95, Z99, rng.uniform(-1.0, 3.0))[rng.integers(4)])
    offset_rows = rng.random() < 0.3
    gate_std = float(np.exp(rng.uniform(np.log(0.1), np.log(10.0))))
    split_ok = rng.random() < 0.8
    return dict(dt=dt, d=d, T=T, in_shift=in_shift, out_shift=out_shift, live=live, z=z,
                offset_rows=offset_rows, gate_std=gate_std, split_ok=split_ok, seed=1000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = draw(i)
    dt, d, T = c["dt"], c["d"], c["T"]
    label = "random %d: %s" % (i, {k: (round(v, 4) if isinstance(v, float) else v) for k, v in c.items()})
    print(label, flush=True)
    if c["offset_rows"]:
        xb = synth.gelu_offset_rows(T, d, seed=c["seed"], dtype=dt)
    else:
        xb = synth.gelu_iid(T, d, seed=c["seed"], dtype=dt, gate_std=c["gate_std"])
    tdt = TORCH_DTYPE[dt]
    flat = torch.full((T * 2 * d + 16,), float("nan"), dtype=tdt, device="cuda")
    x = flat[c["in_shift"]: c["in_shift"] + T * 2 * d].view(T, 2 * d)
    x.copy_(to_device(xb, dt))
    buf, _ = sentinel_buffer(T * d + 16, 1, dt)
    out = buf[c["out_shift"]: c["out_shift"] + T * d].view(tdt).view(T, d)
    live_t = None if c["live"] is None else torch.tensor([c["live"]], dtype=torch.int32, device="cuda")
    ga.gelu_and_mul_sparse(x, c["z"], out=out, live_rows=live_t,
                           workspace=None if c["split_ok"] else False)
    torch.cuda.synchronize()

    everything = bits_of(buf, dt)
    o0 = c["out_shift"]
    outside = np.concatenate([everything[:o0], everything[o0 + T * d:]])
    assert np.all(outside == synth.SENTINEL[dt]), f"{label}: wrote outside the output view"
    got = everything[o0: o0 + T * d].reshape(T, d)
    n = T if c["live"] is None else max(0, min(c["live"], T))
    assert np.all(got[n:] == synth.SENTINEL[dt]), f"{label}: rows beyond the live count were written"
    if n:
        ref, st = oracle.get().gelu_and_mul_sparse(xb[:n], dt, c["z"], want_stats=True)
        compare(got[:n], ref, dt, gate=decode(xb[:n, :d], dt), stats=st, label=label)


N_ELEM_CASES = 200
ELEM_OPS = ("silu", "gelu_tanh", "gelu_erf", "squared_relu")


def draw_elementwise(i):
    rng = np.random.default_rng(104729 * (i + 1))
    op = ELEM_OPS[rng.integers(len(ELEM_OPS))]
    dt = (BF16, F16, F32)[rng.integers(3)]
    d = int(rng.integers(1, 64) if rng.random() < 0.3 else rng.integers(64, 20000))
    if rng.random() < 0.5:
        d = max(8, d // 8 * 8)
    M = max(1, min(int(np.exp(rng.uniform(0.0, np.log(20000.0)))), MAX_ELEMS // d))
    shifted = rng.random() < 0.3
    in_shift = int(rng.integers(0, 4)) if shifted else 0
    out_shift = int(rng.integers(0, 4)) if shifted else 0
    live = int(rng.integers(-2, M + 3)) if (op in ("silu", "squared_relu") or rng.random() < 0.5) else None
    gate_std = float(np.exp(rng.uniform(np.log(0.1), np.log(10.0))))
    return dict(op=op, dt=dt, d=d, M=M, in_shift=in_shift, out_shift=out_shift, live=live, gate_std=gate_std,
                seed=5000 + i)


@pytest.mark.parametrize("i", range(N_ELEM_CASES))
def test_random_elementwise_case(i):
    """silu_and_mul_bounded, gelu_and_mul (tanh and erf) and squared ReLU on
    random shapes, types, shifted views and live counts (negative and past the
    capacity included), planned by the library, against the oracle."""
    c = draw_elementwise(i)
    op, dt, d, M = c["op"], c["dt"], c["d"], c["M"]
    label = "random elementwise %d: %s" % (i, {k: (round(v, 4) if isinstance(v, float) else v)
                                               for k, v in c.items()})
    print(label, flush=True)
    gated = op != "squared_relu"
    xb = synth.gelu_iid(M, d, seed=c["seed"], dtype=dt, gate_std=c["gate_std"])
    if not gated:
        xb = np.ascontiguousarray(xb[:, :d])
    width = xb.shape[1]
    tdt = TORCH_DTYPE[dt]
    flat = torch.full((M * width + 16,), float("nan"), dtype=tdt, device="cuda")
    x = flat[c["in_shift"]: c["in_shift"] + M * width].view(M, width)
    x.copy_(to_device(xb, dt))
    buf, _ = sentinel_buffer(M * d + 16, 1, dt)
    out = buf[c["out_shift"]: c["out_shift"] + M * d].view(tdt).view(M, d)
    live_t = None if c["live"] is None else torch.tensor([c["live"]], dtype=torch.int32, device="cuda")
    o = oracle.get()
    n = M if c["live"] is None else max(0, min(c["live"], M))
    if op == "silu":
        ga.silu_and_mul_bounded(x, live_t, out=out)
        ref = o.silu_and_mul_bounded(xb, dt, n)
    elif op == "squared_relu":
        ga.squared_relu_bounded(x, live_t, out=out)
        ref = o.squared_relu_bounded(xb, dt, n)
    else:
        approx = op == "gelu_tanh"
        ga.gelu_and_mul(x, "tanh" if approx else "none", out=out, live_rows=live_t)
        ref = o.gelu_and_mul(xb, dt, approx, live=n)
    torch.cuda.synchronize()

    everything = bits_of(buf, dt)
    o0 = c["out_shift"]
    outside = np.concatenate([everything[:o0], everything[o0 + M * d:]])
    assert np.all(outside == synth.SENTINEL[dt]), f"{label}: wrote outside the output view"
    got = everything[o0: o0 + M * d].reshape(M, d)
    assert np.all(got[n:] == synth.SENTINEL[dt]), f"{label}: rows beyond the live count were written"
    if n:
        compare(got[:n], ref[:n], dt, label=label)
