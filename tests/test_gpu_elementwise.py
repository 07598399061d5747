"""gelu_and_mul (tanh and erf forms) and the bounded squared ReLU on the GPU
against the fp64 oracle (needs an MI355X).  Both share the elementwise
kernel family of silu_and_mul_bounded: the live count is read on the device,
rows beyond it stay untouched, and the grid depends on the capacity only."""
import numpy as np
import pytest
import torch

import gated_activation_amd as ga
import oracle
import synth
from parity import BF16, F16, F32, bits_of, check_canary, compare, sentinel_buffer, to_device

pytestmark = pytest.mark.gpu


def _live(n):
    return None if n is None else torch.tensor([n], dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("approximate", ["tanh", "none"])
@pytest.mark.parametrize("dt", [F32, F16, BF16], ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("T,d", [(1, 768), (37, 777), (1024, 2048), (64, 8192)])
def test_gelu_and_mul(approximate, dt, T, d):
    xb = synth.gelu_iid(T, d, seed=T + d, dtype=dt, gate_std=2.0)
    o = oracle.get()
    for live in (None, T // 2):
        buf, out = sentinel_buffer(T, d, dt)
        ga.gelu_and_mul(to_device(xb, dt), approximate, out=out, live_rows=_live(live))
        torch.cuda.synchronize()
        check_canary(buf, T, d, dt)
        n = T if live is None else live
        ref = o.gelu_and_mul(xb, dt, approximate == "tanh", live=n)
        got = bits_of(out, dt)
        compare(got[:n], ref[:n], dt, label=f"gelu_and_mul {approximate} dt{dt} T{T} d{d} live{live}")
        assert np.all(got[n:] == synth.SENTINEL[dt])


@pytest.mark.parametrize("approximate", ["tanh", "none"])
def test_gelu_and_mul_saturation(approximate):
    """Large negative gates give -0 (no NaN from an overflowing power); large
    positive ones give the gate itself."""
    d = 64
    g = np.linspace(-60.0, 60.0, 4 * d).reshape(4, d)
    xb = np.concatenate([synth.to_bits(g, F32), synth.to_bits(np.ones_like(g), F32)], axis=1)
    out = ga.gelu_and_mul(to_device(xb, F32), approximate)
    torch.cuda.synchronize()
    ref = oracle.get().gelu_and_mul(xb, F32, approximate == "tanh")
    compare(bits_of(out, F32), ref, F32, label=f"saturation {approximate}")


@pytest.mark.parametrize("dt", [F32, F16, BF16], ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [1, 7, 768, 777, 4096])
def test_squared_relu_bounded(dt, d):
    M = 1000
    xb = synth.to_bits(3.0 * synth.normal(synth.stream_key(d, 5), 0, M * d).reshape(M, d), dt)
    ref = oracle.get().squared_relu_bounded(xb, dt, M)
    x = to_device(xb, dt)
    for live in (0, 1, 500, M, 5000, -7):
        buf, out = sentinel_buffer(M, d, dt)
        ga.squared_relu_bounded(x, _live(live), out=out)
        torch.cuda.synchronize()
        check_canary(buf, M, d, dt)
        n = max(0, min(live, M))
        got = bits_of(out, dt)
        compare(got[:n], ref[:n], dt, label=f"sqrelu dt{dt} d{d} live{live}")
        assert np.all(got[n:] == synth.SENTINEL[dt])


def test_squared_relu_is_exact_on_bf16_squares():
    """relu(x)^2 of a bf16 value with at most 4 significant bits is exact in
    bf16, so the GPU must return exactly the oracle's bits."""
    M, d = 64, 1024
    k = synth.normal(synth.stream_key(3, 9), 0, M * d).reshape(M, d)
    v = np.round(k * 4.0) / 4.0                         # multiples of 1/4, |v| < ~20
    xb = synth.to_bits(v, BF16)
    out = ga.squared_relu_bounded(to_device(xb, BF16), _live(M))
    torch.cuda.synchronize()
    ref = oracle.get().squared_relu_bounded(xb, BF16, M)
    exact = np.abs(v) < 4.0
    assert np.array_equal(bits_of(out, BF16)[exact], ref[exact])


@pytest.mark.parametrize("op", ["silu", "gelu_tanh", "gelu_erf", "sqrelu"])
@pytest.mark.parametrize("dt", [F32, F16, BF16], ids=["f32", "f16", "bf16"])
def test_shifted_views_take_the_unaligned_path(op, dt):
    """Input and output views off a 16-byte boundary (and odd d): the
    unaligned path, 16-byte vectors numbered flat over the output region.
    Elements of the output buffer outside the live part of the view keep
    their sentinel bits; the input view is surrounded by NaN."""
    M = 300
    o = oracle.get()
    tdt = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dt]
    for d in (768, 777, 5):
        cols = 1 if op == "sqrelu" else 2
        if op == "sqrelu":
            xb = synth.to_bits(3.0 * synth.normal(synth.stream_key(d, 11), 0, M * d).reshape(M, d), dt)
        else:
            xb = synth.gelu_iid(M, d, seed=d + 3 * dt, dtype=dt, gate_std=2.0)
        for i_s, o_s in ((1, 0), (0, 1), (3, 5)):
            flat = torch.full((M * cols * d + 16,), float("nan"), dtype=tdt, device="cuda")
            x = flat[i_s: i_s + M * cols * d].view(M, cols * d)
            x.copy_(to_device(xb, dt))
            buf, _ = sentinel_buffer(M * d + 16, 1, dt)
            out = buf[o_s: o_s + M * d].view(tdt).view(M, d)
            for live in (M, 123):
                buf.fill_(int(synth.SENTINEL[dt]))      # below 2^15 / 2^31: the same bits as a signed fill
                lt = _live(live)
                if op == "silu":
                    ga.silu_and_mul_bounded(x, lt, out=out)
                    ref = o.silu_and_mul_bounded(xb, dt, live)
                elif op == "sqrelu":
                    ga.squared_relu_bounded(x, lt, out=out)
                    ref = o.squared_relu_bounded(xb, dt, live)
                else:
                    tanh = op == "gelu_tanh"
                    ga.gelu_and_mul(x, "tanh" if tanh else "none", out=out, live_rows=lt)
                    ref = o.gelu_and_mul(xb, dt, tanh, live=live)
                torch.cuda.synchronize()
                everything = bits_of(buf, dt)
                view = everything[o_s: o_s + M * d].reshape(M, d)
                outside = np.concatenate([everything[:o_s], everything[o_s + M * d:], view[live:].ravel()])
                assert np.all(outside == synth.SENTINEL[dt]), f"{op} d{d} shifts {i_s},{o_s} live {live}: wrote outside"
                compare(view[:live], ref[:live], dt, label=f"{op} dt{dt} d{d} shifts {i_s},{o_s} live {live}")


@pytest.mark.parametrize("dt", [F32, F16, BF16], ids=["f32", "f16", "bf16"])
def test_unaligned_small_d_around_the_vector_width(dt):
    """d from 1 to 17 elements on shifted views: output vectors numbered flat
    over the region straddle several rows (d below a vector), exactly one
    row boundary, or none, and the region's last vector is partial; every
    per-lane count and a grid small enough to loop."""
    M = 37
    o = oracle.get()
    tdt = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dt]
    for d in range(1, 18):
        xb = synth.gelu_iid(M, d, seed=900 + d + 7 * dt, dtype=dt, gate_std=2.0)
        ref = o.silu_and_mul_bounded(xb, dt, M)
        for i_s, o_s in ((1, 2), (3, 0)):
            flat = torch.full((M * 2 * d + 16,), float("nan"), dtype=tdt, device="cuda")
            x = flat[i_s: i_s + M * 2 * d].view(M, 2 * d)
            x.copy_(to_device(xb, dt))
            buf, _ = sentinel_buffer(M * d + 16, 1, dt)
            out = buf[o_s: o_s + M * d].view(tdt).view(M, d)
            for plan in (None, ga.Plan(path=2, per_lane=1, block=256, grid=1),
                         ga.Plan(path=2, per_lane=4, block=256, grid=1)):
                for live in (M, 20):
                    buf.fill_(int(synth.SENTINEL[dt]))
                    ga.silu_and_mul_bounded(x, _live(live), out=out, plan=plan)
                    torch.cuda.synchronize()
                    everything = bits_of(buf, dt)
                    view = everything[o_s: o_s + M * d].reshape(M, d)
                    outside = np.concatenate([everything[:o_s], everything[o_s + M * d:], view[live:].ravel()])
                    label = f"silu dt{dt} d{d} shifts {i_s},{o_s} live {live} plan {plan and plan.per_lane}"
                    assert np.all(outside == synth.SENTINEL[dt]), label + ": wrote outside"
                    compare(view[:live], ref[:live], dt, label=label)
