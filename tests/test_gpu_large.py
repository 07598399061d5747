"""Largest sizes: buffers past 4 GiB (64-bit row offsets), grids past 65535
rows, the largest d, and flat item counts just under the kernels' 2^31 bound.

A block of seeded rows from synth/ is generated on the host and tiled on the
device to the full size.  Rows are independent, so every tile of the output
must be bit-identical to the first (checked on the device), and the first
tile is compared with the oracle on sampled rows.  Rows past a live count
must keep their sentinel bits.
"""
import numpy as np
import pytest
import torch

import gated_activation_amd as ga
import oracle
import synth
from parity import BF16, F16, F32, INT_VIEW, TORCH_DTYPE, Z95, bits_of, compare, decode, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    assert torch.cuda.is_available(), "these tests need a GPU"
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _tiled(block_bits, dtype, reps):
    """[reps * rows, cols] device tensor: the host block repeated."""
    b = to_device(block_bits, dtype)
    return b.repeat(reps, 1)


def _sentinel_out(rows, cols, dtype):
    s = int(synth.SENTINEL[dtype])
    if s >= 1 << (31 if dtype == F32 else 15):
        s -= 1 << (32 if dtype == F32 else 16)
    return torch.full((rows, cols), s, dtype=INT_VIEW[dtype], device="cuda").view(TORCH_DTYPE[dtype])


def _tiles_identical(out, block_rows, n_rows, dtype):
    """Rows [0, n_rows) of out, in tiles of block_rows, all equal tile 0."""
    iv = out.view(INT_VIEW[dtype])
    first = iv[:block_rows]
    for start in range(block_rows, n_rows, block_rows):
        stop = min(start + block_rows, n_rows)
        if not torch.equal(iv[start:stop], first[: stop - start]):
            return start
    return None


def _sentinel_rows_kept(out, start, dtype):
    iv = out.view(INT_VIEW[dtype])[start:]
    s = torch.tensor(int(synth.SENTINEL[dtype]), dtype=torch.int64, device="cuda")
    mask = (1 << (32 if dtype == F32 else 16)) - 1
    return bool(((iv.to(torch.int64) & mask) == s).all())


def test_gelu_sparse_8gib_input_131072_rows():
    """T = 131072, d = 16384, bf16: 8 GiB in, 4 GiB out, grid of 131072 rows."""
    T, d, blk = 131072, 16384, 2048
    xb = synth.gelu_large(blk, d)
    x = _tiled(xb, BF16, T // blk)
    assert x.numel() * 2 > 8 * 2 ** 30 - 1
    out = ga.gelu_and_mul_sparse(x, Z95)
    torch.cuda.synchronize()
    assert _tiles_identical(out, blk, T, BF16) is None
    ref, st = oracle.get().gelu_and_mul_sparse(xb, BF16, Z95, want_stats=True)
    # Every row of the last tile (offsets past 8 GiB in the input).
    got = bits_of(out[T - blk:], BF16)
    compare(got, ref, BF16, gate=decode(xb[:, :d], BF16), stats=st, label="T131072 d16384")


def test_gelu_sparse_largest_d_every_path():
    """d = 65536 (the largest): bf16 on the vector path (16 waves x 8 vectors
    per lane, no split), fp32 on the element path (16 waves x 64 elements)."""
    o = oracle.get()
    for dt, T, blk in ((BF16, 512, 64), (F32, 2048, 32)):
        d = 65536
        xb = synth.gelu_iid(blk, d, seed=65 + dt, dtype=dt, gate_std=1.7)
        x = _tiled(xb, dt, T // blk)
        plan = ga.plan_gelu_and_mul_sparse(T, d, dt, with_workspace=False)
        assert plan.splits == 1 and (plan.path == 0) == (dt == BF16)
        out = ga.gelu_and_mul_sparse(x, Z95, workspace=False)
        torch.cuda.synchronize()
        assert _tiles_identical(out, blk, T, dt) is None
        rows = np.arange(0, blk, 4)
        ref, st = o.gelu_and_mul_sparse(xb[rows], dt, Z95, want_stats=True)
        got = bits_of(out[T - blk + torch.from_numpy(rows).cuda()], dt)
        compare(got, ref, dt, gate=decode(xb[rows, :d], dt), stats=st, label=f"d65536 dt{dt}")
        del x, out


def test_silu_bounded_near_2pow31_elements():
    """M = 2^21 - 4096 rows of d = 1024 bf16: 2.14e9 output elements (the
    bound is rows * d < 2^31), 8 GiB in, live M - 5: the tail rows keep
    their sentinel."""
    M, d, blk = (1 << 21) - 4096, 1024, 4096
    xb = synth.moe_buffer(blk, d, seed=21)
    x = _tiled(xb, BF16, M // blk)
    out = _sentinel_out(M, d, BF16)
    live = torch.tensor([M - 5], dtype=torch.int32, device="cuda")
    ga.silu_and_mul_bounded(x, live, out=out)
    torch.cuda.synchronize()
    assert _tiles_identical(out, blk, M - blk, BF16) is None
    last = out[M - blk: M - 5]
    assert torch.equal(last.view(torch.int16), out[: blk - 5].view(torch.int16))
    assert _sentinel_rows_kept(out, M - 5, BF16)
    rows = np.linspace(0, blk - 1, 32).astype(int)
    ref = oracle.get().silu_and_mul_bounded(xb[rows], BF16, len(rows))
    compare(bits_of(out[torch.from_numpy(rows).cuda()], BF16), ref, BF16, label="silu near 2^31")


def test_squared_relu_unaligned_path_near_2pow31():
    """M = 2^21 rows of d = 1023 fp16 (not 16-byte rows: the unaligned path,
    vectors flat over the output), 2^21 * 1023 = 2.145e9 elements, just under
    the 2^31 bound."""
    M, d, blk = 1 << 21, 1023, 4096
    rng_block = synth.gelu_iid(blk, d, seed=1023, dtype=F16)[:, :d]   # gate half: N(0,1)
    xb = np.ascontiguousarray(rng_block)
    x = _tiled(xb, F16, M // blk)
    plan = ga.plan_silu_and_mul_bounded(M, d, F16)
    assert plan.path == 2
    out = _sentinel_out(M, d, F16)
    live = torch.tensor([M], dtype=torch.int32, device="cuda")
    ga.squared_relu_bounded(x, live, out=out)
    torch.cuda.synchronize()
    assert _tiles_identical(out, blk, M, F16) is None
    rows = np.linspace(0, blk - 1, 32).astype(int)
    ref = oracle.get().squared_relu_bounded(xb[rows], F16, len(rows))
    compare(bits_of(out[M - blk + torch.from_numpy(rows).cuda()], F16), ref, F16, label="sqrelu near 2^31")
