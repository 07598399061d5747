"""Round-trip form of gelu_and_mul_sparse on the GPU against the oracle.

The round-trip form rounds every intermediate to the element type where an
eager PyTorch composition stores a tensor (vLLM PR 48498, section
Cross-architecture warp and dtype validation and the review thread after
it): mean, std, z, z * std, cutoff, gate - cutoff, GELU output, product.
The oracle's `gelu_and_mul_sparse_rt` follows those points in fp64 and is
pinned bit-exactly to torch's eager CPU composition.

What may differ, and how the comparison accounts for it (bf16 / fp16):

* The cutoff.  The GPU reduces the row in fp32, the oracle in fp64; where
  the exact mean or std lies close to a rounding boundary of the element
  type the two may round to neighbouring values.  For each row the test
  bounds the GPU's fp32 statistics (first-order error of a reduction of
  depth at most 128, plus the final roundings), maps the corners of that
  box through the same rounding points (every step is monotone) and takes
  every element-type value between the extreme cutoffs as a candidate.  A
  row passes if it matches the oracle run with one of its candidates.
* The GELU output.  The GPU's fp32 GELU is not correctly rounded, so h may
  land one element-type step from the oracle's; gate - cutoff and the
  product h * up are exact in fp32 for these types and then rounded once on
  both sides.  With h off by one step, |y_gpu - y_oracle| < 3 ulp(y_oracle):
  each rounding contributes half an ulp and ulp(h) * |up| < 2 ulp(y).

fp32 data uses the ordinary comparison (2 ulp / 1e-3 with the exemption
band around the cutoff) against the round-trip oracle.
"""
import numpy as np
import pytest
import torch

import gated_activation_amd as ga
import oracle
import synth
from parity import (BF16, F16, F32, Z95, Z99, bits_of, check_canary, compare, decode,
                    sentinel_buffer, to_device)
from rt_match import cut_candidates, rows_match

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "these tests need a GPU"


def run_rt(x_bits, dtype, z, rows_sample=None, live=None, plan=None, label=""):
    o = oracle.get()
    T, two_d = x_bits.shape
    d = two_d // 2
    x = to_device(x_bits, dtype)
    buf, out = sentinel_buffer(T, d, dtype)
    live_t = None if live is None else torch.tensor([live], dtype=torch.int32, device="cuda")
    if plan is None:
        ga.gelu_and_mul_sparse(x, z, out=out, live_rows=live_t, round_intermediates=True)
    else:
        plan.flags = ga.GA_ROUND_INTERMEDIATES
        ga.gelu_and_mul_sparse(x, z, out=out, live_rows=live_t, plan=plan)
    torch.cuda.synchronize()
    got = bits_of(out, dtype)
    check_canary(buf, T, d, dtype)
    n = T if live is None else max(0, min(live, T))
    assert np.all(got[n:] == synth.SENTINEL[dtype]), f"{label}: rows beyond the live count were written"
    rows = np.arange(n) if rows_sample is None else np.array(sorted(set(rows_sample)), int)
    rows = rows[rows < n]
    if rows.size == 0:
        return {}
    xs = x_bits[rows]
    ref, st = o.gelu_and_mul_sparse_rt(xs, dtype, z)
    gate = decode(xs[:, :d], dtype)
    if dtype == F32:
        return compare(got[rows], ref, dtype, gate=gate, stats=st, label=label)

    cands = cut_candidates(o, gate, dtype, z)
    unresolved = [i for i, c in enumerate(cands) if c is None]
    assert len(unresolved) <= max(1, rows.size // 100), f"{label}: {len(unresolved)} rows too ambiguous"
    for i, c in enumerate(cands):
        if c is not None:
            assert st[2][i] in c, f"{label}: row {rows[i]}: oracle cutoff {st[2][i]!r} not among {c}"
    g_rows = got[rows]
    # Candidate 0 is the oracle's own cutoff; the others exist only where
    # the row is ambiguous.
    order = [[st[2][i]] + [v for v in c if v != st[2][i]] if c is not None else [st[2][i]]
             for i, c in enumerate(cands)]
    m0 = rows_match(g_rows, ref, dtype)
    # Bit-exactness over the rows that took the oracle's own cutoff.
    bitexact_frac = float((g_rows[m0] == ref[m0]).mean()) if m0.any() else 1.0
    ok = m0.copy()
    for j in range(1, max(len(c) for c in order)):
        cut_j = np.array([c[min(j, len(c) - 1)] for c in order])
        ok |= rows_match(g_rows, o.gelu_and_mul_sparse_rt(xs, dtype, z, cut=cut_j)[0], dtype)
    bad = [i for i in np.flatnonzero(~ok) if i not in unresolved]
    assert not bad, (f"{label}: rows {[int(rows[i]) for i in bad[:5]]} match no candidate cutoff "
                     f"(oracle cut {[float(st[2][i]) for i in bad[:5]]})")
    n_alt = int((~m0).sum())
    res = {"rows": int(rows.size), "rows_other_candidate": n_alt, "bitexact_frac": bitexact_frac,
           "ambiguous_rows": int(sum(1 for c in cands if c is not None and len(c) > 1)),
           "unresolved": len(unresolved)}
    print(f"{label}: {res}", flush=True)
    return res


def test_small_check_case_bf16():
    """T=4, d=2048, bf16, gate/up N(0,1), seed 0."""
    res = run_rt(synth.gelu_iid(4, 2048, seed=0), BF16, Z95, label="rt T4 d2048")
    assert res["bitexact_frac"] > 0.99


@pytest.mark.parametrize("T", [1, 7, 128, 2048])
def test_token_sweep_d8192(T):
    """Gate N(0,1) + per-row offset N(0,0.5), seed = T; at T = 2048 the
    oracle checks 96 sampled rows."""
    x = synth.gelu_offset_rows(T, 8192)
    sample = None if T <= 128 else list(np.linspace(0, T - 1, 96).astype(int))
    res = run_rt(x, BF16, Z95, rows_sample=sample, label=f"rt sweep T{T}")
    assert res["bitexact_frac"] > 0.99
    assert res["rows_other_candidate"] <= max(1, res["rows"] // 5)


@pytest.mark.parametrize("dt", [BF16, F16, F32], ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [1, 31, 128, 4096, 16384])
def test_dtypes_and_sizes(dt, d):
    """The page's small d (1, 31, 128; odd d takes the unaligned path) and larger rows."""
    T = 64 if d <= 4096 else 16
    x = synth.gelu_iid(T, d, seed=d + 17 * dt, dtype=dt)
    res = run_rt(x, dt, Z95, label=f"rt {dt} d{d}")
    if dt != F32 and d >= 128:
        assert res["bitexact_frac"] > 0.98


@pytest.mark.parametrize("dt", [BF16, F16, F32], ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("z", [0.0, Z95, Z99], ids=["z0", "z95", "z99"])
def test_edge_mix(dt, z):
    """Near-constant, constant (drawn, 0, 100) and Student-t(3) rows."""
    x = synth.edge_rows(25, 2048, dt)
    run_rt(x, dt, z, label=f"rt edge {dt} z{z}")


def test_live_rows():
    x = synth.gelu_iid(64, 2048, seed=5)
    for live in (0, 1, 37, 64, 1000, -3):
        run_rt(x, BF16, Z95, live=live, label=f"rt live {live}")


@pytest.mark.parametrize("geom", [(0, 16, 1, 0), (0, 8, 2, 0), (0, 4, 4, 1), (0, 2, 8, 1), (1, 16, 16, 0),
                                  (2, 8, 3, 0), (2, 4, 5, 0), (2, 8, 2, 1)],
                         ids=lambda g: f"path{g[0]}_w{g[1]}_pl{g[2]}_late{g[3]}")
def test_every_geometry(geom):
    """The form is the same for any launch geometry of d = 8192 bf16."""
    path, w, pl, late = geom
    plan = ga.Plan(path=path, waves_per_row=w, per_lane=pl, up_late=late, block=64 * w)
    run_rt(synth.gelu_offset_rows(32, 8192), BF16, Z95, plan=plan, label=f"rt geom {geom}")


@pytest.mark.parametrize("dt", [BF16, F16], ids=["bf16", "f16"])
def test_packed_rows(dt):
    """Short rows, several per wavefront (the packed-rows kernels)."""
    for d, g, v in ((64, 4, 2), (128, 8, 2), (256, 16, 2), (256, 32, 1)):
        x = synth.gelu_offset_rows(203, d, seed=700 + d, dtype=dt)
        plan = ga.Plan(path=3, lanes_per_row=g, per_lane=v, block=256)
        res = run_rt(x, dt, Z95, plan=plan, label=f"rt packed dt{dt} d{d} g{g} v{v}")
        assert res["bitexact_frac"] > 0.98


def test_round_trip_differs_from_default_as_the_pages_describe():
    """On bf16 the rounded cutoff moves the threshold by up to half a bf16
    step of the cutoff, so the two forms disagree on some elements; both
    forms must still each match their own oracle."""
    x_bits = synth.gelu_iid(64, 4096, seed=11)
    x = to_device(x_bits, BF16)
    a = ga.gelu_and_mul_sparse(x, Z95)
    b = ga.gelu_and_mul_sparse(x, Z95, round_intermediates=True)
    torch.cuda.synchronize()
    diff = (bits_of(a, BF16) != bits_of(b, BF16)).mean()
    assert 0.0 < diff < 0.5


@pytest.mark.parametrize("i", range(128))
def test_random_cases(i):
    """Seeded random shapes, types, z, gate scales and live counts through the
    planner's own choice, against the round-trip oracle as above."""
    rng = np.random.default_rng(15485863 * (i + 1))
    dt = (BF16, F16, F32)[rng.integers(3)]
    d = int(rng.integers(1, 300) if rng.random() < 0.3 else rng.integers(300, 20000))
    if rng.random() < 0.5:
        d = max(8, d // 8 * 8)
    T = max(1, min(int(np.exp(rng.uniform(0.0, np.log(2000.0)))), 500_000 // d))
    z = float((0.0, Z95, Z99, rng.uniform(-1.0, 3.0))[rng.integers(4)])
    live = None if rng.random() < 0.6 else int(rng.integers(0, T + 3))
    gate_std = float(np.exp(rng.uniform(np.log(0.1), np.log(10.0))))
    xb = synth.gelu_iid(T, d, seed=9000 + i, dtype=dt, gate_std=gate_std)
    run_rt(xb, dt, z, live=live, label=f"rt random {i}: dt{dt} T{T} d{d} z{z:.4f} live{live} std{gate_std:.3f}")
