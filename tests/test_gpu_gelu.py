"""gelu_and_mul_sparse on the GPU against the fp64 oracle (needs an MI355X).

Cases follow the workloads on the pages (vLLM PR 48498: token counts 1-2048,
intermediate sizes 2048-32768, small d = 1, 31, 128 over fp16/bf16/fp32),
with seeded synthetic rows (synth/): the small check case, the d = 8192 token
sweep with per-row offsets, large rows up to d = 32768, and the edge mix
(variance cancellation, constant rows, Student-t(3) tails, odd d, three z).
"""
import numpy as np
import pytest
import torch

import gated_activation_amd as ga
import oracle
import synth
from parity import (BF16, F16, F32, TORCH_DTYPE, Z95, Z99, bits_of, check_canary, compare,
                    decode, sentinel_buffer, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"
    props = torch.cuda.get_device_properties(0)
    print(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}",
          flush=True)


def run_and_check(x_bits, dtype, z, rows_sample=None, plan=None, live=None, label=""):
    """GPU call on the whole input; oracle on all rows (or the sampled ones)."""
    o = oracle.get()
    T, two_d = x_bits.shape
    d = two_d // 2
    x = to_device(x_bits, dtype)
    buf, out = sentinel_buffer(T, d, dtype)
    live_t = None if live is None else torch.tensor([live], dtype=torch.int32, device="cuda")
    ga.gelu_and_mul_sparse(x, z, out=out, live_rows=live_t, plan=plan)
    torch.cuda.synchronize()
    got = bits_of(out, dtype)
    check_canary(buf, T, d, dtype)
    n = T if live is None else max(0, min(live, T))
    rows = np.arange(n) if rows_sample is None else np.array(sorted(set(rows_sample)) if n else [], int)
    rows = rows[rows < n]
    if rows.size:
        ref, st = o.gelu_and_mul_sparse(x_bits[rows], dtype, z, want_stats=True)
        gate = decode(x_bits[rows, :d], dtype)
        res = compare(got[rows], ref, dtype, gate=gate, stats=st, label=label)
    else:
        res = {}
    assert np.all(got[n:] == synth.SENTINEL[dtype]), f"{label}: rows beyond the live count were written"
    return res


def test_small_check_case():
    """T=4, d=2048, bf16, gate/up N(0,1), seed 0, z = Phi^-1(0.95)."""
    x = synth.gelu_iid(4, 2048, seed=0)
    res = run_and_check(x, BF16, Z95, label="T4 d2048")
    assert res["bitexact_frac"] > 0.99


@pytest.mark.parametrize("T", [1, 2, 8, 32, 128, 512, 2048])
def test_token_sweep_d8192(T):
    """Gate N(0,1) + per-row offset N(0,0.5), up N(0,1), seed = T."""
    x = synth.gelu_offset_rows(T, 8192)
    run_and_check(x, BF16, Z95, label=f"sweep T{T}")


@pytest.mark.parametrize("d", [16384, 32768])
@pytest.mark.parametrize("T", [1, 64, 2048])
def test_large_rows(T, d):
    """Gate N(0,2), up N(0,1): 32 KB and 64 KB gate rows.  Every row is
    compared with the oracle, the benchmark's own shape (T = 2048,
    d = 16384) and T = 2048, d = 32768 included."""
    x = synth.gelu_large(T, d)
    run_and_check(x, BF16, Z95, label=f"large T{T} d{d}")


@pytest.mark.parametrize("z", [0.0, Z95, Z99], ids=["z0", "z95", "z99"])
@pytest.mark.parametrize("T", [1, 7, 333])
@pytest.mark.parametrize("d", [2000, 3000, 8191])
@pytest.mark.parametrize("dt", [F16, BF16], ids=["f16", "bf16"])
def test_edge_mix(dt, d, T, z):
    x = synth.edge_rows(T, d, dt)
    run_and_check(x, dt, z, label=f"edge dt{dt} d{d} T{T} z{z}")


@pytest.mark.parametrize("z", [0.0, Z95])
@pytest.mark.parametrize("d", [1, 31, 128])
@pytest.mark.parametrize("dt", [F32, F16, BF16], ids=["f32", "f16", "bf16"])
def test_small_d_all_dtypes(dt, d, z):
    x = synth.gelu_iid(5, d, seed=100 + d, dtype=dt, gate_std=1.5)
    run_and_check(x, dt, z, label=f"small dt{dt} d{d}")


@pytest.mark.parametrize("dt", [F32, F16])
def test_other_dtypes_large(dt):
    x = synth.gelu_iid(96, 8192, seed=55, dtype=dt, gate_std=2.0)
    run_and_check(x, dt, Z95, label=f"dt{dt} T96 d8192")


@pytest.mark.parametrize("live", [0, 1, 37, 64, 100, -3])
def test_live_rows_bound(live):
    x = synth.gelu_iid(64, 2048, seed=7)
    run_and_check(x, BF16, Z95, live=live, label=f"live {live}")


def _all_vector_plans(d, dtype):
    per16 = 4 if dtype == F32 else 8
    for w in (1, 2, 4, 8, 16):
        for v in (1, 2, 4, 8):
            if w * 64 * v * per16 >= d:
                for late in (0, 1):
                    yield ga.Plan(path=0, waves_per_row=w, per_lane=v, up_late=late, block=64 * w, grid=0)


def test_every_vector_geometry_matches_oracle():
    """Every compiled vector geometry that covers the row gives an
    oracle-matching result (reduction order differs between them)."""
    x = synth.gelu_offset_rows(24, 8192, seed=77)
    for p in _all_vector_plans(8192, BF16):
        run_and_check(x, BF16, Z95, plan=p, label=f"plan w{p.waves_per_row} v{p.per_lane} late{p.up_late}")


# Shapes at which the planner's measured rule picks each of its row
# geometries: (T, d) -> (waves, vectors per lane, up late).
# Shapes where the planner's measured table picks different row geometries
# (1 to 16 waves, 1 to 8 vectors per lane, up early and late).
PLANNER_SHAPES = [(1024, 1024), (8192, 1024), (2048, 2048), (4096, 2048), (3072, 1600), (1024, 4096),
                  (2048, 4096), (900, 5600), (512, 16384), (4096, 16384), (512, 32768), (256, 32768),
                  (640, 20480), (384, 24576), (2048, 14336), (4096, 12288), (1800, 4800)]


@pytest.mark.parametrize("T,d", PLANNER_SHAPES, ids=[f"T{t}-d{d}" for t, d in PLANNER_SHAPES])
def test_planner_geometry_at_its_shapes(T, d):
    """The default call at shapes across the planner's geometry choices, on
    sampled rows (first, last and scattered) against the oracle."""
    p = ga.plan_gelu_and_mul_sparse(T, d, BF16)
    assert (p.path, p.splits) == (0, 1) or p.path == 4
    print(f"T={T} d={d}: path {p.path}, waves {p.waves_per_row}, vectors per lane {p.per_lane}, "
          f"up late {p.up_late}, splits {p.splits}", flush=True)
    x = synth.gelu_offset_rows(T, d, seed=T * 7 + d)
    rng = np.random.default_rng(T + d)
    sample = list(range(16)) + list(range(T - 16, T)) + list(rng.integers(0, T, 32))
    run_and_check(x, BF16, Z95, rows_sample=sample, label=f"planner T{T} d{d}")


def test_element_path_on_aligned_rows():
    x = synth.gelu_offset_rows(24, 4096, seed=78)
    for w, e in ((1, 64), (4, 16), (16, 4), (4, 64), (16, 16)):
        p = ga.Plan(path=1, waves_per_row=w, per_lane=e, block=64 * w, grid=0)
        run_and_check(x, BF16, Z95, plan=p, label=f"elem w{w} e{e}")


@pytest.mark.parametrize("shift", [1, 3, 7])
def test_misaligned_base_pointers(shift):
    """Bases off 16-byte alignment by `shift` elements (the unaligned path)."""
    T, d = 9, 2048
    xb = synth.gelu_iid(T, d, seed=shift)
    flat = torch.zeros(T * 2 * d + 16, dtype=torch.bfloat16, device="cuda")
    x = flat[shift: shift + T * 2 * d].view(T, 2 * d)
    x.copy_(to_device(xb, BF16))
    buf = torch.zeros(T * d + 16, dtype=torch.bfloat16, device="cuda")
    out = buf[shift: shift + T * d].view(T, d)
    ga.gelu_and_mul_sparse(x, Z95, out=out)
    torch.cuda.synchronize()
    o = oracle.get()
    ref, st = o.gelu_and_mul_sparse(xb, BF16, Z95, want_stats=True)
    compare(bits_of(out, BF16), ref, BF16, gate=decode(xb[:, :d], BF16), stats=st, label="misaligned")
    assert not bits_of(buf[:shift], BF16).any() and not bits_of(buf[shift + T * d:], BF16).any()


def run_offset(xb, dt, z, in_shift, out_shift, plan=None, rows_sample=None, label=""):
    """Input and output views that start in_shift / out_shift elements past a
    16-byte boundary; every element of the output buffer outside the view
    must keep its sentinel bits."""
    T, two_d = xb.shape
    d = two_d // 2
    tdt = TORCH_DTYPE[dt]
    # NaN around the input view: a read past the view would bring NaN into
    # the statistics or the output.
    flat = torch.full((T * two_d + 16,), float("nan"), dtype=tdt, device="cuda")
    x = flat[in_shift: in_shift + T * two_d].view(T, two_d)
    x.copy_(to_device(xb, dt))
    buf, _ = sentinel_buffer(T * d + 16, 1, dt)
    out = buf[out_shift: out_shift + T * d].view(tdt).view(T, d)
    ga.gelu_and_mul_sparse(x, z, out=out, plan=plan)
    torch.cuda.synchronize()
    everything = bits_of(buf, dt)
    outside = np.concatenate([everything[:out_shift], everything[out_shift + T * d:]])
    assert np.all(outside == synth.SENTINEL[dt]), f"{label}: wrote outside the output view"
    rows = np.arange(T) if rows_sample is None else np.array(sorted(set(rows_sample)), int)
    ref, st = oracle.get().gelu_and_mul_sparse(xb[rows], dt, z, want_stats=True)
    got = everything[out_shift: out_shift + T * d].reshape(T, d)[rows]
    return compare(got, ref, dt, gate=decode(xb[rows, :d], dt), stats=st, label=label)


@pytest.mark.parametrize("dt", [BF16, F16, F32], ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [1, 5, 31, 1000, 8191, 16383, 16384])
def test_unaligned_path_every_phase_mix(dt, d):
    """Rows off a 16-byte boundary (shifted bases, odd d: phases change from
    row to row) take the unaligned path; input and output shifts vary
    independently.  With odd d every row but the last reads its partial last
    up vector whole (into the next row) and the last row element by element;
    tiny d (1, 5) also reads the gate's partial vector element by element near
    the end of the buffer."""
    T = 37 if d <= 8191 else 9
    xb = synth.gelu_iid(T, d, seed=300 + d + dt, dtype=dt, gate_std=1.4)
    per = 4 if dt == F32 else 8
    for i_s, o_s in ((0, 1), (1, 0), (3, 3), (per - 1, 2 % per), (1, per - 1)):
        if d % per == 0 and i_s == 0 and o_s == 0:
            continue
        plan = ga.plan_gelu_and_mul_sparse(T, d, dt, aligned=False)
        assert plan.path == (3 if d * (16 // per) <= 512 else 2)    # short rows are packed
        run_offset(xb, dt, Z95, i_s, o_s, label=f"unaligned dt{dt} d{d} shifts {i_s},{o_s}")


def test_unaligned_path_every_geometry():
    """Every unaligned-path geometry that covers the row, with up loaded
    early or late, on shifted and on aligned rows, matches the oracle."""
    d = 8191
    xb = synth.gelu_offset_rows(12, d, seed=79)
    nvec = (d + 7) // 8
    for w in (1, 2, 4, 8, 16):
        for v in range(1, 9):
            if w * 64 * v < nvec:
                continue
            for late in (0, 1):
                p = ga.Plan(path=2, waves_per_row=w, per_lane=v, up_late=late, block=64 * w)
                for i_s, o_s in ((0, 0), (5, 2), (2, 5)):
                    run_offset(xb, BF16, Z95, i_s, o_s, plan=p,
                               label=f"unaligned w{w} v{v} late{late} shifts {i_s},{o_s}")


@pytest.mark.parametrize("dt,d", [(BF16, 16384), (F16, 8192), (F32, 4096)], ids=["bf16", "f16", "f32"])
def test_unaligned_path_is_bit_identical_to_vector_path_on_aligned_rows(dt, d):
    """On 16-byte rows the unaligned path holds the same vectors in the same
    lanes as the vector path, so with the same geometry the bytes match."""
    T = 64
    xb = synth.gelu_iid(T, d, seed=d + dt, dtype=dt, gate_std=1.3)
    x = to_device(xb, dt)
    for w, v, late in ((8, (d * (4 if dt == F32 else 2)) // 16 // 512, 1), (16, 2 if dt != F32 else 1, 0)):
        if w * 64 * v * (16 // (4 if dt == F32 else 2)) < d:
            continue
        outs = []
        for path in (0, 2):
            p = ga.Plan(path=path, waves_per_row=w, per_lane=v, up_late=late, block=64 * w)
            outs.append(bits_of(ga.gelu_and_mul_sparse(x, Z95, plan=p), dt))
        torch.cuda.synchronize()
        assert np.array_equal(outs[0], outs[1]), (w, v, late)


def test_unaligned_path_headline_rows():
    """T = 2048, d = 16384 bf16 one element off alignment, every row."""
    xb = synth.gelu_large(2048, 16384)
    run_offset(xb, BF16, Z95, 1, 1, label="unaligned headline")


def _packed_plans(d, dt):
    per = 4 if dt == F32 else 8
    nvec = -(-d // per)
    for g in (4, 8, 16, 32):
        for v in (1, 2, 4):
            if g * v >= nvec and g * (v // 2 if v > 1 else 0) < nvec:
                yield ga.Plan(path=3, lanes_per_row=g, per_lane=v, block=256)


# Rows of at most 32 16-byte vectors (fp32: d <= 128) are the packed path's.
PACKED_CASES = [(d, dt) for dt in (BF16, F16, F32) for d in (8, 64, 128, 256) if d * (4 if dt == F32 else 2) <= 512]
PACKED_IDS = [f"{d}-{ {BF16: 'bf16', F16: 'f16', F32: 'f32'}[dt]}" for d, dt in PACKED_CASES]


@pytest.mark.parametrize("d,dt", PACKED_CASES, ids=PACKED_IDS)
def test_packed_rows_every_geometry(dt, d):
    """Short aligned rows, several per wavefront: every packed geometry that
    covers the row, with T leaving a ragged last workgroup, matches the
    oracle; so does the planner's choice at a large T."""
    T = 203
    x = synth.gelu_offset_rows(T, d, seed=500 + d + dt, dtype=dt)
    plans = list(_packed_plans(d, dt))
    assert plans
    for p in plans:
        run_and_check(x, dt, Z95, plan=p, label=f"packed dt{dt} d{d} g{p.lanes_per_row} v{p.per_lane}")
    big = synth.gelu_iid(9000, d, seed=d, dtype=dt)
    assert ga.plan_gelu_and_mul_sparse(9000, d, dt).path == 3
    run_and_check(big, dt, Z95, rows_sample=list(range(0, 9000, 97)) + [8999], label=f"packed big dt{dt} d{d}")


@pytest.mark.parametrize("live", [0, 1, 63, 64, 65, 200, 203, 10 ** 6, -1])
def test_packed_rows_live_bound(live):
    """Live counts that end inside, at and past a workgroup's rows."""
    x = synth.gelu_iid(203, 128, seed=17)
    run_and_check(x, BF16, Z95, live=live, label=f"packed live {live}")


def test_packed_rows_edge_and_constant_rows():
    for dt in (BF16, F16):
        x = synth.edge_rows(40, 256, dt, seed=8)
        for z in (0.0, Z95, Z99):
            run_and_check(x, dt, z, label=f"packed edge dt{dt} z{z}")


PACKED_UNA_CASES = [(d, dt) for dt in (BF16, F16, F32) for d in (1, 3, 7, 9, 31, 64, 100, 127, 255, 256)
                    if d * (4 if dt == F32 else 2) <= 512]
PACKED_UNA_IDS = [f"{d}-{ {BF16: 'bf16', F16: 'f16', F32: 'f32'}[dt]}" for d, dt in PACKED_UNA_CASES]


@pytest.mark.parametrize("d,dt", PACKED_UNA_CASES, ids=PACKED_UNA_IDS)
def test_packed_rows_unaligned(dt, d):
    """Short rows off 16-byte alignment (shifted views, odd d) packed several
    per wavefront: every covering geometry, input and output shifts varied
    independently, NaN around the input view.  Rows of 1 and 3 elements read
    their last gate vector element by element near the end of the buffer."""
    es = 4 if dt == F32 else 2
    per = 16 // es
    T = 203
    xb = synth.gelu_offset_rows(T, d, seed=700 + d + dt, dtype=dt)
    plans = list(_packed_plans(d, dt))
    assert plans
    for p in plans:
        for i_s, o_s in ((0, 1), (1, 0), (per - 1, per - 1), (3, 2 % per), (0, 0)):
            if d % per == 0 and i_s == 0 and o_s == 0:
                continue
            run_offset(xb, dt, Z95, i_s, o_s, plan=p,
                       label=f"packed unaligned dt{dt} d{d} g{p.lanes_per_row} v{p.per_lane} shifts {i_s},{o_s}")


@pytest.mark.parametrize("live", [0, 1, 31, 32, 33, 200, 203, 10 ** 6, -1])
def test_packed_rows_unaligned_live_bound(live):
    """Odd d on a shifted view, packed: live counts that end inside, at and
    past a workgroup's rows (16 rows of 16 lanes per workgroup); rows past
    the count keep their sentinel bits."""
    T, d = 203, 127
    xb = synth.gelu_iid(T, d, seed=23)
    flat = torch.full((T * 2 * d + 8,), float("nan"), dtype=torch.bfloat16, device="cuda")
    x = flat[5: 5 + T * 2 * d].view(T, 2 * d)
    x.copy_(to_device(xb, BF16))
    buf, _ = sentinel_buffer(T * d + 8, 1, BF16)
    out = buf[3: 3 + T * d].view(torch.bfloat16).view(T, d)
    assert ga.plan_gelu_and_mul_sparse(T, d, BF16).path == 3
    live_t = torch.tensor([live], dtype=torch.int32, device="cuda")
    ga.gelu_and_mul_sparse(x, Z95, out=out, live_rows=live_t)
    torch.cuda.synchronize()
    everything = bits_of(buf, BF16)
    n = max(0, min(live, T))
    got = everything[3: 3 + T * d].reshape(T, d)
    assert np.all(everything[:3] == synth.SENTINEL[BF16]) and np.all(everything[3 + T * d:] == synth.SENTINEL[BF16])
    assert np.all(got[n:] == synth.SENTINEL[BF16]), "rows past the live count were written"
    if n:
        ref, st = oracle.get().gelu_and_mul_sparse(xb[:n], BF16, Z95, want_stats=True)
        compare(got[:n], ref, BF16, gate=decode(xb[:n, :d], BF16), stats=st, label=f"packed unaligned live {live}")


@pytest.mark.parametrize("dt", [BF16, F16])
def test_packed_rows_unaligned_planner_and_edge_rows(dt):
    """The planner's packed choice on shifted views at a large T (sampled
    rows), and the edge mix (cancellation, constant rows, heavy tails) on an
    odd d."""
    big = synth.gelu_iid(9000, 255, seed=41 + dt, dtype=dt)
    assert ga.plan_gelu_and_mul_sparse(9000, 255, dt).path == 3
    run_offset(big, dt, Z95, 3, 5, rows_sample=list(range(0, 9000, 89)) + [8999], label=f"packed big dt{dt}")
    x = synth.edge_rows(40, 255, dt, seed=9)
    for z in (0.0, Z95, Z99):
        run_offset(x, dt, z, 1, 2, label=f"packed edge unaligned dt{dt} z{z}")


@pytest.mark.parametrize("dt,d", [(BF16, 128), (F16, 256), (F32, 64)], ids=["bf16", "f16", "f32"])
def test_packed_rows_unaligned_is_bit_identical_to_aligned(dt, d):
    """On rows of whole 16-byte vectors, shifted bases give the same vectors
    in the same lanes as aligned ones, so the bytes match."""
    T = 300
    xb = synth.gelu_iid(T, d, seed=d + 3 * dt, dtype=dt, gate_std=1.3)
    tdt = TORCH_DTYPE[dt]
    for p in _packed_plans(d, dt):
        ref = bits_of(ga.gelu_and_mul_sparse(to_device(xb, dt), Z95, plan=p), dt)
        flat = torch.zeros(T * 2 * d + 8, dtype=tdt, device="cuda")
        x = flat[3: 3 + T * 2 * d].view(T, 2 * d)
        x.copy_(to_device(xb, dt))
        obuf = torch.zeros(T * d + 8, dtype=tdt, device="cuda")
        out = obuf[1: 1 + T * d].view(T, d)
        ga.gelu_and_mul_sparse(x, Z95, out=out, plan=p)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out, dt), ref), (p.lanes_per_row, p.per_lane)


def test_repeat_runs_are_bit_identical():
    x = to_device(synth.gelu_large(64, 16384), BF16)
    a = ga.gelu_and_mul_sparse(x, Z95)
    b = ga.gelu_and_mul_sparse(x, Z95)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_constant_rows_give_exact_zeros():
    T, d = 6, 16384
    vals = np.array([0.0, 100.0, -3.5, 1e-3, 7.25, -250.0])
    xb = np.concatenate([synth.to_bits(np.repeat(vals[:, None], d, 1), BF16),
                         synth.to_bits(np.ones((T, d)), BF16)], axis=1)
    for z in (0.0, Z95):
        out = ga.gelu_and_mul_sparse(to_device(xb, BF16), z)
        torch.cuda.synchronize()
        assert np.all(decode(bits_of(out, BF16), BF16) == 0.0)


@pytest.mark.parametrize("dt,tiny", [(F16, 2.0 ** -20), (BF16, 2.0 ** -130), (F32, 2.0 ** -140)],
                         ids=["f16", "bf16", "f32"])
def test_subnormal_outputs_are_rounded_not_flushed(dt, tiny):
    """One element passes the cutoff (hand-worked row: gate 0,...,0,8) and up
    is a subnormal of the type, so the exact output is subnormal too: it must
    round to nearest even like the oracle, not flush to zero."""
    gate = np.array([0.0] * 7 + [8.0])
    up = np.full(8, tiny)
    xb = np.concatenate([synth.to_bits(gate, dt), synth.to_bits(up, dt)])[None, :]
    out = ga.gelu_and_mul_sparse(to_device(xb, dt), Z95)
    torch.cuda.synchronize()
    ref = oracle.get().gelu_and_mul_sparse(xb, dt, Z95)
    got = bits_of(out, dt)
    assert decode(ref, dt)[0, 7] != 0.0
    assert np.array_equal(got, ref), (got, ref)


# ---------------------------------------------------------------------------
# Few long rows shared by several workgroups: split rows (partial statistics
# exchanged through the workspace) or replicated statistics, as planned.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,d", [(1, 16384), (8, 16384), (64, 16384), (1, 32768), (64, 32768),
                                 (128, 32768), (3, 65536), (8, 32768), (16, 32768), (4, 65536)])
def test_few_rows_default_plan(T, d):
    p = ga.plan_gelu_and_mul_sparse(T, d, ga.GA_BF16)
    assert p.splits > 1
    print(f"T={T} d={d}: path {p.path} splits {p.splits}", flush=True)
    x = synth.gelu_large(T, d)
    run_and_check(x, BF16, Z95, label=f"few rows T{T} d{d} path{p.path}")


def _tiling_plans(nvec):
    """Every split plan whose chunks tile a row of nvec vectors: S = ceil(nvec /
    chunk) workgroups, each owning at least one vector."""
    for w in (1, 2, 4, 8, 16):
        for v in (1, 2, 4):
            chunk = w * 64 * v
            S = -(-nvec // chunk)
            if 2 <= S <= 16:
                yield ga.Plan(path=0, waves_per_row=w, per_lane=v, block=64 * w, splits=S)


def test_split_rows_every_split_count():
    """Split counts 2..16, uneven counter shares included (rows of 1024, 1100
    and 1600 vectors), give oracle-matching output."""
    seen = set()
    for d in (8192, 8800, 12800):
        x = synth.gelu_offset_rows(6, d, seed=91)
        for p in _tiling_plans(d // 8):
            seen.add(p.splits)
            run_and_check(x, BF16, Z95, plan=p, label=f"d{d} S{p.splits} w{p.waves_per_row} v{p.per_lane}")
    assert seen >= {2, 3, 4, 5, 7, 8, 9, 13, 16}, seen


def test_split_rows_forced_fallback():
    """With a poll bound of zero every workgroup computes the whole row's
    statistics itself: the result must still match the oracle."""
    x = synth.gelu_large(8, 32768)
    p = ga.plan_gelu_and_mul_sparse(8, 32768, ga.GA_BF16)
    assert p.path == 0 and p.splits > 1
    p.spin_limit = 0
    run_and_check(x, BF16, Z95, plan=p, label="fallback")
    q = ga.Plan(path=0, waves_per_row=4, per_lane=2, splits=4, block=256, spin_limit=0)
    run_and_check(synth.gelu_large(8, 16384), BF16, Z95, plan=q, label="fallback 4 splits")


def test_split_workspace_reused_across_shapes():
    """One workspace serves calls of different T and split counts in any
    order (each call tags all of a row's slots with the previous call's tag
    plus 16)."""
    ws = torch.zeros(ga.lib.ga_gelu_and_mul_sparse_workspace_bytes(128), dtype=torch.uint8, device="cuda")
    o = oracle.get()
    shapes = ((8, 16384, 4), (2, 8800, 3), (128, 32768, 2), (8, 12800, 7), (64, 16384, 16),
              (1, 32768, 8), (3, 8800, 9))
    for T, d, S in shapes:
        xb = synth.gelu_iid(T, d, seed=T * 7 + S, gate_std=1.3)
        nvec = d // 8
        plan = next(p for p in _tiling_plans(nvec) if p.splits == S)
        out = ga.gelu_and_mul_sparse(to_device(xb, BF16), Z95, plan=plan, workspace=ws)
        torch.cuda.synchronize()
        ref, st = o.gelu_and_mul_sparse(xb, BF16, Z95, want_stats=True)
        compare(bits_of(out, BF16), ref, BF16, gate=decode(xb[:, :d], BF16), stats=st, label=f"reuse T{T} S{S}")
    # Each row's record: 16 slots of two 64-bit words {tag, value}.  After any
    # sequence of calls all 32 tags of a row are equal (the tag of the row's
    # last call, a multiple of 16; 0 for rows never processed).
    tags = ws.view(torch.int32).cpu().numpy().reshape(128, 32, 2)[:, :, 0]
    assert np.all(tags == tags[:, :1])
    # Row r was processed by every call with T > r, each adding 16.
    calls = np.array([T for T, _, _ in shapes])
    want = 16 * (calls[None, :] > np.arange(128)[:, None]).sum(axis=1)
    assert np.array_equal(tags[:, 0], want), (tags[:, 0], want)


@pytest.mark.parametrize("live", [0, 3, 8, 20])
def test_split_rows_live_bound(live):
    x = synth.gelu_large(8, 32768)
    run_and_check(x, BF16, Z95, live=live, label=f"split live {live}")


@pytest.mark.parametrize("dt,d", [(F16, 32768), (F32, 16384), (F16, 16384)], ids=["f16", "f32", "f16-rep"])
def test_split_rows_other_dtypes(dt, d):
    x = synth.gelu_iid(4, d, seed=123, dtype=dt, gate_std=2.0)
    p = ga.plan_gelu_and_mul_sparse(4, d, dt)
    assert p.splits > 1 and p.path == (4 if d * (4 if dt == F32 else 2) == 32768 else 0)
    run_and_check(x, dt, Z95, label=f"few rows dt{dt} d{d} path{p.path}")


def test_split_rows_constant_and_edge_rows():
    """Constant rows still give exact zeros through the partial combine;
    near-constant N(100, 0.01) and Student-t rows match the oracle."""
    split = ga.Plan(path=0, waves_per_row=4, per_lane=2, splits=4, block=256)
    for dt in (F16, BF16):
        x = synth.edge_rows(10, 16384, dt, seed=5)
        assert ga.plan_gelu_and_mul_sparse(10, 16384, dt).splits > 1
        for z in (0.0, Z95):
            run_and_check(x, dt, z, label=f"few rows edge dt{dt} z{z}")
            run_and_check(x, dt, z, plan=split, label=f"split edge dt{dt} z{z}")
    T, d = 5, 32768
    vals = np.array([0.0, 100.0, -3.5, 7.25, -250.0])
    xb = np.concatenate([synth.to_bits(np.repeat(vals[:, None], d, 1), BF16),
                         synth.to_bits(np.ones((T, d)), BF16)], axis=1)
    out = ga.gelu_and_mul_sparse(to_device(xb, BF16), 0.0)
    torch.cuda.synchronize()
    assert np.all(decode(bits_of(out, BF16), BF16) == 0.0)


# Few rows, statistics replicated: `splits` workgroups per row, each reducing
# the whole gate row and applying its share (no workspace).
def _rep_plans(d, dt):
    per16 = 4 if dt == F32 else 8
    nvec = d // per16
    for w in (1, 2, 4, 8, 16):
        for v in (1, 2, 4, 8):
            if nvec <= w * 64 * v < 8 * nvec:
                for rep in (2, 4, 8):
                    yield ga.Plan(path=4, waves_per_row=w, per_lane=v, splits=rep, block=64 * w)


@pytest.mark.parametrize("dt,d", [(BF16, 8192), (BF16, 2048), (F16, 8192), (F32, 4096), (BF16, 16384)],
                         ids=["bf16-8192", "bf16-2048", "f16-8192", "f32-4096", "bf16-16384"])
def test_replicated_statistics_every_geometry(dt, d):
    """Every replicated-statistics geometry matches the oracle, writes only
    its rows (T = 13: a ragged group of 8 rows), and is bit-identical to the
    one-row kernel with the same waves and vectors (the same reduction), so
    all shares of a row used the same cutoff."""
    T = 13
    x = synth.gelu_offset_rows(T, d, seed=900 + d + dt, dtype=dt)
    xd = to_device(x, dt)
    plans = list(_rep_plans(d, dt))
    assert plans
    for p in plans:
        run_and_check(x, dt, Z95, plan=p, label=f"rep dt{dt} d{d} w{p.waves_per_row} v{p.per_lane} s{p.splits}")
        one = ga.Plan(path=0, waves_per_row=p.waves_per_row, per_lane=p.per_lane, up_late=0, block=p.block)
        a = bits_of(ga.gelu_and_mul_sparse(xd, Z95, plan=p), dt)
        b = bits_of(ga.gelu_and_mul_sparse(xd, Z95, plan=one), dt)
        torch.cuda.synchronize()
        assert np.array_equal(a, b), (p.waves_per_row, p.per_lane, p.splits)


@pytest.mark.parametrize("live", [0, 1, 5, 8, 9, 13, 100, -2])
def test_replicated_statistics_live_rows(live):
    """Live counts inside, at and past a group of 8 rows leave the other rows
    untouched."""
    x = synth.gelu_offset_rows(13, 8192, seed=31)
    p = ga.Plan(path=4, waves_per_row=8, per_lane=2, splits=4, block=512)
    run_and_check(x, BF16, Z95, plan=p, live=live, label=f"rep live {live}")
