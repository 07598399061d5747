"""silu_and_mul_bounded on the GPU against the fp64 oracle (needs an MI355X).

Megatron-LM PR 6328 ("Size MoE activation kernel grid to the row count"):
a capture-sized MoE buffer of M rows, a device-side live count, and rows
beyond it left untouched.  The op is elementwise with no cross-workgroup
reduction, so every launch geometry must give byte-identical output.
"""
import numpy as np
import pytest
import torch

import gated_activation_amd as ga
import oracle
import synth
from parity import BF16, F16, F32, bits_of, check_canary, compare, sentinel_buffer, to_device

pytestmark = pytest.mark.gpu

M, D = 16384, 768


@pytest.fixture(scope="module")
def moe():
    xb = synth.moe_buffer(M, D)
    ref = oracle.get().silu_and_mul_bounded(xb, BF16, M)
    return xb, to_device(xb, BF16), ref


def run(x, live, dtype, M_, d, plan=None):
    buf, out = sentinel_buffer(M_, d, dtype)
    live_t = torch.tensor([live], dtype=torch.int32, device="cuda")
    ga.silu_and_mul_bounded(x, live_t, out=out, plan=plan)
    torch.cuda.synchronize()
    check_canary(buf, M_, d, dtype)
    return bits_of(out, dtype)


@pytest.mark.parametrize("live", [64, 512, 1024, 4096, 16384])
def test_moe_decode_buffer(moe, live):
    """M = 16384, d = 768, bf16 N(0,1); sentinel rows beyond the live count."""
    xb, x, ref = moe
    got = run(x, live, BF16, M, D)
    compare(got[:live], ref[:live], BF16, label=f"silu live {live}")
    assert np.all(got[live:] == synth.SENTINEL[BF16])


@pytest.mark.parametrize("live,n", [(0, 0), (-5, 0), (M + 100, M), (2 ** 31 - 1, M)])
def test_live_count_is_clamped(moe, live, n):
    xb, x, ref = moe
    got = run(x, live, BF16, M, D)
    compare(got[:n], ref[:n], BF16, label=f"clamp {live}")
    assert np.all(got[n:] == synth.SENTINEL[BF16])


def test_every_geometry_is_byte_identical(moe):
    xb, x, ref = moe
    live = 3001
    base = run(x, live, BF16, M, D)
    for pl in (1, 2, 4):
        for grid in (1, 7, 256, 2048, 6144):
            p = ga.Plan(path=0, waves_per_row=0, per_lane=pl, block=256, grid=grid)
            assert np.array_equal(run(x, live, BF16, M, D, plan=p), base), (pl, grid)
    for pl in (1, 4):
        p = ga.Plan(path=1, waves_per_row=0, per_lane=pl, block=256, grid=512)
        assert np.array_equal(run(x, live, BF16, M, D, plan=p), base), ("elem", pl)
    for pl in (1, 2, 4):
        for grid in (1, 512, 4096):
            p = ga.Plan(path=2, waves_per_row=0, per_lane=pl, block=256, grid=grid)
            assert np.array_equal(run(x, live, BF16, M, D, plan=p), base), ("unaligned", pl, grid)


@pytest.mark.parametrize("dt", [F32, F16, BF16], ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [1, 5, 777, 1024, 4096])
def test_other_shapes_and_dtypes(dt, d):
    Mx = 300
    xb = synth.moe_buffer(Mx, d, seed=d, dtype=dt)
    ref = oracle.get().silu_and_mul_bounded(xb, dt, Mx)
    for live in (0, 1, 123, Mx):
        got = run(to_device(xb, dt), live, dt, Mx, d)
        compare(got[:live], ref[:live], dt, label=f"silu dt{dt} d{d} live{live}")
        assert np.all(got[live:] == synth.SENTINEL[dt])


def test_large_magnitudes_saturate_cleanly():
    """silu(g) -> 0 for g << 0 and -> g for g >> 0, with no NaN."""
    d = 64
    g = np.linspace(-120.0, 120.0, 4 * d).reshape(4, d)
    xb = np.concatenate([synth.to_bits(g, F32), synth.to_bits(np.ones_like(g), F32)], axis=1)
    ref = oracle.get().silu_and_mul_bounded(xb, F32, 4)
    got = run(to_device(xb, F32), 4, F32, 4, d)
    compare(got, ref, F32, label="saturation")
