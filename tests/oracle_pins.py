"""Pins for the fp64 oracle: checks against things other than the oracle.

Each pin takes an `oracle.Oracle` and raises AssertionError when the oracle
disagrees with an independent source: numpy's float casts, an exhaustive
nearest-value search, torch's fp64 GELU / SiLU routines, numpy's mean and
std, exact rational arithmetic, closed forms, invariances of the definition,
and the Gaussian survival fraction 1 - Phi(z).  The planted-mistake test runs
every pin against edited copies of the oracle and requires each edit to be
caught by at least one of them.

Definitions pinned (vLLM PR 48498, "Purpose"; Megatron-LM PR 6328, "What
changed and why"): per row, cutoff = mean + z * population std of the gate,
out = gelu_tanh(relu(gate - cutoff)) * up, rounded once to the output type;
silu_and_mul_bounded: out = silu(gate) * up on live rows only.
"""
import math
from fractions import Fraction

import numpy as np
import torch

import synth
from oracle import BF16, F16, F32

Z95 = float(np.float32(1.6448536))
Z99 = float(np.float32(2.3263479))


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# element codec
# ---------------------------------------------------------------------------

def _all_bf16_as_f64():
    bits = np.arange(1 << 16, dtype=np.uint32)
    return bits.astype(np.uint16), (bits << np.uint32(16)).view(np.float32).astype(np.float64)


def pin_decode(o):
    # fp16: every bit pattern against numpy's float16.
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = o.decode(bits, F16)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m]), "fp16 decode"
    assert np.array_equal(np.signbit(got[m]), np.signbit(ref[m]))
    # bf16: every bit pattern against the top half of an IEEE binary32.
    b16, ref = _all_bf16_as_f64()
    got = o.decode(b16, BF16)
    m = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[m], ref[m]), "bf16 decode"
    # fp32: random patterns plus the specials.
    r = _rng(1).integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    r = np.concatenate([r, np.array([0, 0x80000000, 1, 0x007FFFFF, 0x00800000,
                                     0x7F7FFFFF, 0x7F800000, 0xFF800000], np.uint32)])
    ref = r.view(np.float32).astype(np.float64)
    got = o.decode(r, F32)
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m]), "fp32 decode"


def _encode_probe_values(rng, lo_exp, hi_exp, n=100000):
    """Random doubles over a range of binades, both signs, plus exact ties."""
    e = rng.integers(lo_exp, hi_exp, n)
    v = np.ldexp(rng.random(n) + 1.0, e) * np.where(rng.random(n) < 0.5, -1.0, 1.0)
    return v


def pin_encode_fp32(o):
    rng = _rng(2)
    v = _encode_probe_values(rng, -160, 130)
    # exact midpoints between adjacent floats: tie cases
    f = rng.standard_normal(20000).astype(np.float32)
    nxt = np.nextafter(f, np.float32(np.inf))
    mids = (f.astype(np.float64) + nxt.astype(np.float64)) / 2.0
    v = np.concatenate([v, mids, [0.0, -0.0, 3.5e38, -3.5e38, 1e-46, 7e-46]])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float32).view(np.uint32)
    got = o.encode(v, F32)
    assert np.array_equal(got, ref), "fp32 encode vs IEEE cast"


def pin_encode_fp16(o):
    rng = _rng(3)
    v = _encode_probe_values(rng, -30, 17)
    h = rng.standard_normal(20000).astype(np.float16)
    nxt = np.nextafter(h, np.float16(np.inf))
    mids = (h.astype(np.float64) + nxt.astype(np.float64)) / 2.0
    sub = rng.random(5000) * 6.2e-5          # subnormal range
    v = np.concatenate([v, mids, sub, -sub, [65504.0, 65519.99, 65520.0, 1e6, -1e6]])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = o.encode(v, F16)
    assert np.array_equal(got, ref), "fp16 encode vs numpy"


def _nearest_bf16_bits(v):
    """Exhaustive nearest search over all finite bf16 values, ties to the even
    (last mantissa bit 0) one, overflow past the last midpoint to inf."""
    bits, vals = _all_bf16_as_f64()
    pos = (vals >= 0) & np.isfinite(vals) & ~np.signbit(vals)
    pbits, pvals = bits[pos], vals[pos]
    order = np.argsort(pvals)
    pbits, pvals = pbits[order], pvals[order]
    a = np.abs(v)
    idx = np.clip(np.searchsorted(pvals, a), 1, len(pvals) - 1)
    lo, hi = pvals[idx - 1], pvals[idx]
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & ((pbits[idx] & 1) == 0))
    out = np.where(pick_hi, pbits[idx], pbits[idx - 1]).astype(np.uint32)
    top = pvals[-1]
    half_ulp_top = 2.0 ** (127 - 8)          # overflow threshold: top + half an ulp
    out = np.where(a >= top + half_ulp_top, np.uint32(0x7F80), out)
    sign = np.signbit(v).astype(np.uint32) << np.uint32(15)
    return (out | sign).astype(np.uint16)


def pin_encode_bf16(o):
    rng = _rng(4)
    v = _encode_probe_values(rng, -140, 128, 60000)
    _, vals = _all_bf16_as_f64()
    fin = vals[np.isfinite(vals)]
    fin = np.unique(fin)
    mids = (fin[:-1] + fin[1:]) / 2.0
    mids = mids[np.isfinite(mids)]
    v = np.concatenate([v, rng.choice(mids, 20000), [0.0, -0.0, 3.4e38, 3.40e38 * 1.001, 1e-40]])
    got = o.encode(v, BF16)
    ref = _nearest_bf16_bits(v)
    assert np.array_equal(got, ref), "bf16 encode vs exhaustive nearest-even search"
    # One rounding straight from double: 1 + 2^-8 + 2^-30 lies above the
    # midpoint of 1 and 1 + 2^-7; a detour through fp32 would land on the
    # midpoint and tie down to 1.0.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert int(o.encode(np.array([x]), BF16)[0]) == 0x3F81
    assert int(o.encode(np.array([-x]), BF16)[0]) == 0xBF81


def pin_roundtrip(o):
    for dt in (F16, BF16):
        bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        v = o.decode(bits, dt)
        m = ~np.isnan(v)
        assert np.array_equal(o.encode(v[m], dt), bits[m])


# ---------------------------------------------------------------------------
# elementwise functions
# ---------------------------------------------------------------------------

def pin_gelu(o):
    s = np.concatenate([np.linspace(0.0, 12.0, 4001), [1e-8, 1e-3, 30.0, 100.0]])
    got = o.gelu_tanh(s)
    ref = torch.nn.functional.gelu(torch.from_numpy(s), approximate="tanh").numpy()
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300), "gelu vs torch tanh gelu"
    # Negative side (unused by the op, but part of the function): 1 + tanh
    # cancels there, so the agreement is looser.
    s = np.linspace(-3.0, 0.0, 601)
    ref = torch.nn.functional.gelu(torch.from_numpy(s), approximate="tanh").numpy()
    assert np.allclose(o.gelu_tanh(s), ref, rtol=1e-11, atol=1e-300)
    assert o.gelu_tanh(np.array([0.0]))[0] == 0.0
    # The tanh form approximates x * Phi(x); on [0, 10] the two differ by at
    # most about 4.73e-4 (attained near x = 2.7), a fingerprint of the
    # constants sqrt(2/pi) and 0.044715.
    x = np.linspace(0.0, 10.0, 200001)
    erf_form = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    dev = np.abs(o.gelu_tanh(x) - erf_form)
    assert 4.6e-4 < dev.max() < 4.8e-4, dev.max()
    assert 2.5 < x[np.argmax(dev)] < 2.9


def pin_silu(o):
    x = np.concatenate([np.linspace(-40.0, 40.0, 8001), [0.0, 700.0, -700.0, 1e-9]])
    got = o.silu(x)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300), "silu vs torch silu"
    # silu(x) - silu(-x) = x(sigmoid(x) + sigmoid(-x)) = x
    y = np.linspace(-20, 20, 401)
    assert np.allclose(o.silu(y) - o.silu(-y), y, rtol=1e-13, atol=1e-13)
    assert o.silu(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# row statistics
# ---------------------------------------------------------------------------

def pin_row_stats(o):
    rng = _rng(5)
    for d in (1, 2, 7, 128, 2000, 8191):
        g = rng.standard_normal(d) * 3.0 + 1.5
        mean, std = o.row_stats(g)
        assert math.isclose(mean, float(np.mean(g)), rel_tol=1e-12, abs_tol=1e-13)
        assert math.isclose(std, float(np.std(g, ddof=0)), rel_tol=1e-12, abs_tol=1e-13)
    # Arithmetic progression a + b*i: mean a + b(d-1)/2, variance b^2 (d^2-1)/12.
    for a, b, d in ((0.0, 1.0, 8), (-3.0, 0.25, 1000), (10.0, -2.0, 4097)):
        g = a + b * np.arange(d, dtype=np.float64)
        mean, std = o.row_stats(g)
        assert math.isclose(mean, a + b * (d - 1) / 2.0, rel_tol=1e-14, abs_tol=1e-12)
        assert math.isclose(std, abs(b) * math.sqrt((d * d - 1) / 12.0), rel_tol=1e-13)
    # Exact rationals on bf16-valued rows of 8.
    _, vals = _all_bf16_as_f64()
    fin = vals[np.isfinite(vals) & (np.abs(vals) < 1e4) & (np.abs(vals) > 1e-4)]
    for _ in range(50):
        g = rng.choice(fin, 8)
        fr = [Fraction(float(x)) for x in g]
        mu = sum(fr) / 8
        var = sum((x - mu) ** 2 for x in fr) / 8
        mean, std = o.row_stats(g)
        assert math.isclose(mean, float(mu), rel_tol=1e-15, abs_tol=1e-15)
        assert math.isclose(std, math.sqrt(float(var)), rel_tol=1e-13)
    # A constant row has zero spread; d = 1 likewise.
    assert o.row_stats(np.full(333, 2.75)) == (2.75, 0.0)
    assert o.row_stats(np.array([5.0]))[1] == 0.0


# ---------------------------------------------------------------------------
# whole operations
# ---------------------------------------------------------------------------

def _torch_gelu_sparse_f64(gate, up, z):
    g = torch.from_numpy(gate)
    mean = g.mean(dim=1, keepdim=True)
    std = g.std(dim=1, keepdim=True, correction=0)
    s = torch.relu(g - (mean + z * std))
    return (torch.nn.functional.gelu(s, approximate="tanh") * torch.from_numpy(up)).numpy()


def pin_gelu_sparse_composition(o):
    """Whole op (unrounded) against torch fp64 library routines."""
    for dt, d, T, z, seed in ((BF16, 2000, 6, Z95, 11), (F16, 128, 9, Z99, 12),
                              (F32, 31, 5, 0.0, 13), (BF16, 7, 16, 0.5, 14),
                              (F16, 4096, 3, Z95, 15)):
        x = synth.gelu_iid(T, d, seed=seed, dtype=dt, gate_std=1.7)
        y, f64, st = o.gelu_and_mul_sparse(x, dt, z, want_f64=True, want_stats=True)
        gate = o.decode(x[:, :d], dt)
        up = o.decode(x[:, d:], dt)
        ref = _torch_gelu_sparse_f64(gate, up, z)
        # Summation order differs from torch's (pairwise): the cutoff agrees to
        # ~1e-15 relative, which near the cutoff is an absolute error ~1e-14.
        assert np.allclose(f64, ref, rtol=1e-12, atol=1e-12), (dt, d, T)
        assert np.array_equal(y, o.encode(f64, dt))
        assert np.allclose(st[0], gate.mean(1), rtol=1e-13, atol=1e-14)
        assert np.allclose(st[1], gate.std(1), rtol=1e-12, atol=1e-14)
        assert np.allclose(st[2], gate.mean(1) + z * gate.std(1), rtol=1e-12, atol=1e-13)


def pin_gelu_sparse_invariants(o):
    rng = _rng(6)
    T, d = 8, 512
    x = synth.gelu_iid(T, d, seed=21, dtype=BF16)
    y, f64, st = o.gelu_and_mul_sparse(x, BF16, Z95, want_f64=True, want_stats=True)
    gate = o.decode(x[:, :d], BF16)
    up = o.decode(x[:, d:], BF16)
    # The mask is exactly gate > cutoff, wherever up is nonzero.
    nz = up != 0
    assert np.array_equal((f64 != 0)[nz], (gate > st[2][:, None])[nz])
    # Linear in up: doubling up (exact in bf16) doubles every output.
    x2 = x.copy()
    x2[:, d:] = synth.to_bits(2.0 * up, BF16)
    f2 = o.gelu_and_mul_sparse(x2, BF16, Z95, want_f64=True)[1]
    assert np.array_equal(f2, 2.0 * f64)
    # The up half does not move the mask: replacing it changes no zero pattern.
    x3 = x.copy()
    x3[:, d:] = synth.to_bits(np.ones((T, d)), BF16)
    f3 = o.gelu_and_mul_sparse(x3, BF16, Z95, want_f64=True)[1]
    assert np.array_equal(f3 != 0, gate > st[2][:, None])
    # Scaling the gate by 2^3 scales mean, std and cutoff exactly: same mask.
    x4 = x.copy()
    x4[:, :d] = synth.to_bits(8.0 * gate, BF16)
    f4 = o.gelu_and_mul_sparse(x4, BF16, Z95, want_f64=True)[1]
    assert np.array_equal((f4 != 0)[nz], (f64 != 0)[nz])
    # Shifting the gate by a constant keeps the mask (fp32 rows of multiples
    # of 1/64, so the shifted values are exact).
    gq = np.round(gate * 64.0) / 64.0
    xs = np.concatenate([synth.to_bits(gq, F32), synth.to_bits(up, F32)], axis=1)
    xt = np.concatenate([synth.to_bits(gq + 4.0, F32), synth.to_bits(up, F32)], axis=1)
    assert np.array_equal(o.decode(xt[:, :d], F32), gq + 4.0)
    fs = o.gelu_and_mul_sparse(xs, F32, Z95, want_f64=True)[1]
    ft = o.gelu_and_mul_sparse(xt, F32, Z95, want_f64=True)[1]
    assert np.array_equal((fs != 0)[nz], (ft != 0)[nz])
    assert 0 < (fs != 0).sum() < fs.size
    # Constant rows give zeros at every z; d = 1 gives zero.
    for z in (0.0, Z95, Z99):
        xc = np.empty((3, 2 * 100), np.uint16)
        xc[:, :100] = synth.to_bits(np.array([[0.0], [100.0], [-1.25]]) * np.ones((1, 100)), BF16)
        xc[:, 100:] = synth.to_bits(rng.standard_normal((3, 100)), BF16)
        assert np.all(o.decode(o.gelu_and_mul_sparse(xc, BF16, z), BF16) == 0)
        x1 = synth.to_bits(np.array([[3.0, 7.0], [-2.0, 1.0]]), F16)
        assert np.all(o.decode(o.gelu_and_mul_sparse(x1, F16, z), F16) == 0)
    # Rows at and beyond the live count are not written.
    sentinel = np.full((T, d), synth.SENTINEL[BF16])
    part = o.gelu_and_mul_sparse(x, BF16, Z95, live=3, out=sentinel)
    assert np.array_equal(part[:3], y[:3]) and np.all(part[3:] == synth.SENTINEL[BF16])
    assert np.all(o.gelu_and_mul_sparse(x, BF16, Z95, live=-5, out=sentinel) == sentinel)
    assert np.array_equal(o.gelu_and_mul_sparse(x, BF16, Z95, live=99), y)


def _phi_sf(z):
    return 0.5 * math.erfc(z / math.sqrt(2.0))


def pin_survival_fraction(o):
    """For Gaussian gates a fraction 1 - Phi(z) of elements pass the cutoff."""
    T, d = 64, 8192
    x = synth.gelu_iid(T, d, seed=31, dtype=BF16)
    up_nz = o.decode(x[:, d:], BF16) != 0
    for z, tol in ((Z95, 2.5e-3), (Z99, 1.2e-3), (0.0, 5e-3)):
        f64 = o.gelu_and_mul_sparse(x, BF16, z, want_f64=True)[1]
        frac = (f64 != 0).sum() / up_nz.sum()
        assert abs(frac - _phi_sf(z)) < tol, (z, frac, _phi_sf(z))
    # Scale and shift do not change it: per-row offsets N(0, 0.5).
    x = synth.gelu_offset_rows(32, 8192, seed=32)
    f64 = o.gelu_and_mul_sparse(x, BF16, Z95, want_f64=True)[1]
    frac = (f64 != 0).mean()
    assert abs(frac - _phi_sf(Z95)) < 3e-3, frac


def _brute_1x8(gate, up, z):
    """Exact rational mean and variance, then the textbook formula in Python
    floats: the hand-worked 1x8 rows."""
    fr = [Fraction(float(v)) for v in gate]
    mu = sum(fr) / len(fr)
    var = sum((v - mu) ** 2 for v in fr) / len(fr)
    c = float(mu) + z * math.sqrt(float(var))
    out = []
    for g, u in zip(gate, up):
        s = max(float(g) - c, 0.0)
        h = 0.5 * s * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (s + 0.044715 * s ** 3)))
        out.append(h * float(u))
    return np.array(out)


def pin_brute_force_1x8(o):
    cases = [
        ([0, 0, 0, 0, 0, 0, 0, 8], [1] * 8, Z95),
        ([1, 2, 3, 4, 5, 6, 7, 8], [1, -1, 2, -2, 0.5, -0.5, 4, -4], Z95),
        ([1, 2, 3, 4, 5, 6, 7, 8], [1, -1, 2, -2, 0.5, -0.5, 4, -4], 0.0),
        ([-1, 1, -1, 1, -1, 1, -1, 1], [1, 2, 3, 4, 5, 6, 7, 8], 0.0),
    ]
    rng = _rng(7)
    for _ in range(40):
        cases.append((list(rng.integers(-16, 17, 8) / 4.0), list(rng.standard_normal(8)),
                      float(rng.choice([0.0, Z95, Z99, 0.3]))))
    for gate, up, z in cases:
        z = float(np.float32(z))      # z crosses the boundary as a float
        for dt in (BF16, F16):
            x = np.concatenate([synth.to_bits(np.array(gate, float), dt),
                                synth.to_bits(np.array(up, float), dt)])[None, :]
            g = o.decode(x[0, :8], dt)
            u = o.decode(x[0, 8:], dt)
            ref = _brute_1x8(g, u, z)
            y, f64 = o.gelu_and_mul_sparse(x, dt, z, want_f64=True)
            assert np.allclose(f64[0], ref, rtol=1e-13, atol=1e-15), (gate, up, z)
            with np.errstate(over="ignore"):
                if dt == F16:
                    assert np.array_equal(y[0], ref.astype(np.float16).view(np.uint16))
    # Hand-worked row A: only the last element passes; out = gelu_tanh(8 - c).
    x = np.concatenate([synth.to_bits(np.array([0.0] * 7 + [8.0]), BF16),
                        synth.to_bits(np.ones(8), BF16)])[None, :]
    y = o.decode(o.gelu_and_mul_sparse(x, BF16, Z95), BF16)[0]
    assert np.all(y[:7] == 0) and y[7] == 2.640625


def pin_silu_bounded(o):
    M, d = 40, 96
    for dt in (BF16, F16, F32):
        xb = synth.moe_buffer(M, d, seed=41, dtype=dt)
        sentinel = np.full((M, d), synth.SENTINEL[dt])
        for live in (0, 1, 17, M, M + 5, -3):
            y, f64 = o.silu_and_mul_bounded(xb, dt, live, out=sentinel, want_f64=True)
            n = max(0, min(live, M))
            g = torch.from_numpy(o.decode(xb[:n, :d], dt))
            u = torch.from_numpy(o.decode(xb[:n, d:], dt))
            ref = (torch.nn.functional.silu(g) * u).numpy()
            assert np.allclose(f64[:n], ref, rtol=1e-14, atol=1e-300)
            assert np.array_equal(y[:n], o.encode(f64[:n], dt))
            assert np.all(y[n:] == synth.SENTINEL[dt])


def pin_gelu_erf(o):
    x = np.linspace(0.0, 12.0, 2401)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.allclose(o.gelu_erf(x), ref, rtol=1e-14, atol=1e-300), "erf gelu vs torch"
    y = np.linspace(-6.0, 0.0, 601)          # 1 + erf cancels on this side
    ref = torch.nn.functional.gelu(torch.from_numpy(y), approximate="none").numpy()
    assert np.allclose(o.gelu_erf(y), ref, rtol=1e-8, atol=1e-300)
    # x Phi(x) - (-x) Phi(-x) = x (Phi(x) + Phi(-x)) = x;  gelu(1) = Phi(1).
    z = np.linspace(-8.0, 8.0, 321)
    assert np.allclose(o.gelu_erf(z) - o.gelu_erf(-z), z, rtol=1e-13, atol=1e-13)
    assert math.isclose(o.gelu_erf(np.array([1.0]))[0], 0.5 * math.erfc(-1.0 / math.sqrt(2.0)), rel_tol=1e-15)
    assert o.gelu_erf(np.array([0.0]))[0] == 0.0


def pin_squared_relu(o):
    x = np.concatenate([np.linspace(-5.0, 5.0, 1001), [0.0, -0.0, 1e-200, 1e150]])
    got = o.squared_relu(x)
    ref = (torch.nn.functional.relu(torch.from_numpy(x)) ** 2).numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(o.squared_relu(2.0 * x[:1001]), 4.0 * got[:1001])   # degree-2 homogeneous
    assert np.all(got[x <= 0] == 0.0)


def pin_gelu_and_mul(o):
    for dt, T, d, seed in ((BF16, 7, 333, 51), (F16, 5, 64, 52), (F32, 3, 1000, 53)):
        x = synth.gelu_iid(T, d, seed=seed, dtype=dt, gate_std=2.5)
        g = torch.from_numpy(o.decode(x[:, :d], dt))
        u = torch.from_numpy(o.decode(x[:, d:], dt))
        for approximate, mode in ((True, "tanh"), (False, "none")):
            y, f64 = o.gelu_and_mul(x, dt, approximate, want_f64=True)
            ref = (torch.nn.functional.gelu(g, approximate=mode) * u).numpy()
            # Negative gates: 1 + tanh(w) (or 1 + erf) cancels; both sides then
            # agree to an absolute ~1e-16 |gate|, not relatively.
            assert np.allclose(f64, ref, rtol=1e-12, atol=1e-13), (dt, mode)
            assert np.array_equal(y, o.encode(f64, dt))
        ta = o.gelu_and_mul(x, dt, True, want_f64=True)[1]
        te = o.gelu_and_mul(x, dt, False, want_f64=True)[1]
        assert 1e-5 < np.abs(ta - te).max() < 1e-2 * np.abs(o.decode(x[:, d:], dt)).max()
        sentinel = np.full((T, d), synth.SENTINEL[dt])
        part = o.gelu_and_mul(x, dt, False, live=2, out=sentinel)
        assert np.all(part[2:] == synth.SENTINEL[dt])
        assert np.array_equal(part[:2], o.gelu_and_mul(x, dt, False)[:2])


def pin_squared_relu_bounded(o):
    M, d = 30, 257
    for dt in (BF16, F16, F32):
        x = synth.to_bits(3.0 * synth.normal(synth.stream_key(61, 1), 0, M * d).reshape(M, d), dt)
        ref = (torch.nn.functional.relu(torch.from_numpy(o.decode(x, dt))) ** 2).numpy()
        sentinel = np.full((M, d), synth.SENTINEL[dt])
        for live in (0, 11, M, M + 3, -1):
            y, f64 = o.squared_relu_bounded(x, dt, live, out=sentinel, want_f64=True)
            n = max(0, min(live, M))
            assert np.array_equal(f64[:n], ref[:n])
            assert np.array_equal(y[:n], o.encode(ref[:n], dt))
            assert np.all(y[n:] == synth.SENTINEL[dt])


def _torch_eager_sparse(x_bits, d, dtype, z):
    """The op as native torch composes it on tensors of the element type:
    every intermediate tensor holds that type."""
    tdt = {BF16: torch.bfloat16, F16: torch.float16, F32: torch.float32}[dtype]
    view = np.int32 if dtype == F32 else np.int16
    xt = torch.from_numpy(np.ascontiguousarray(x_bits).view(view)).view(tdt)
    g, u = xt[:, :d], xt[:, d:]
    mean = g.mean(-1, keepdim=True)
    std = g.std(-1, keepdim=True, correction=0)
    cut = mean + std * torch.tensor(z, dtype=torch.float32).to(tdt)
    y = torch.nn.functional.gelu(torch.relu(g - cut), approximate="tanh") * u
    bits = y.contiguous().view(torch.int32 if dtype == F32 else torch.int16).numpy()
    return bits.view(np.uint32 if dtype == F32 else np.uint16), cut.float().numpy()[:, 0]


def pin_gelu_sparse_roundtrip(o):
    """Round-trip form against torch's eager composition in the element type
    (torch rounds every op's result to the tensor type)."""
    cases = [(BF16, synth.gelu_offset_rows(48, 2048, seed=71), 2048, Z95),
             (F16, synth.gelu_iid(32, 4096, seed=72, dtype=F16, gate_std=1.5), 4096, Z99),
             (BF16, synth.edge_rows(15, 3000, BF16, seed=73), 3000, 0.0),
             (F16, synth.edge_rows(15, 2000, F16, seed=74), 2000, Z95),
             (F32, synth.gelu_iid(8, 1024, seed=75, dtype=F32), 1024, Z95)]
    for dt, x, d, z in cases:
        y, st = o.gelu_and_mul_sparse_rt(x, dt, z)
        ref, cut = _torch_eager_sparse(x, d, dt, z)
        if dt == F32:
            # torch's fp32 statistics and tanh are not correctly rounded: the
            # cutoffs agree to an ulp or so and the outputs to ~1e-7.
            assert np.allclose(cut, st[2], rtol=1e-6, atol=1e-6)
            assert np.allclose(o.decode(y, dt), o.decode(ref, dt), rtol=1e-5, atol=1e-6)
            continue
        assert np.array_equal(cut, st[2]), (dt, d)
        assert (y == ref).mean() > 0.9999, (dt, d, (y == ref).mean())
        yd, rd = o.decode(y, dt), o.decode(ref, dt)
        ulp = np.abs(rd) * 2.0 ** -(8 if dt == BF16 else 11) + 2.0 ** -24
        assert np.all(np.abs(yd - rd) <= 2 * ulp)
    # The rounded multiplier moves the cutoff: bf16 holds z = 1.6448536 as
    # 1.6484375, so the round-trip result differs from the one-rounding form.
    x = synth.gelu_iid(16, 2048, seed=76)
    assert not np.array_equal(o.gelu_and_mul_sparse_rt(x, BF16, Z95)[0], o.gelu_and_mul_sparse(x, BF16, Z95))
    assert float(o.decode(o.encode(np.array([Z95]), BF16), BF16)[0]) == 1.6484375
    # A supplied cutoff replaces the computed one.
    y1, st1 = o.gelu_and_mul_sparse_rt(x, BF16, Z95)
    y2, st2 = o.gelu_and_mul_sparse_rt(x, BF16, 0.0, cut=st1[2])
    assert np.array_equal(y1, y2) and np.array_equal(st1[2], st2[2])



# ---------------------------------------------------------------------------
# the activation followed by the down projection
# ---------------------------------------------------------------------------

def pin_down_projection(o):
    """y = a . w^T with a the stored activation: exact rational sums on tiny
    inputs (nearest bf16 by exhaustive search), numpy's fp64 product at a
    moderate size, single-weight and permutation weights that pick out one
    activation element exactly (a transposed operand or output fails), and
    rows beyond the live count untouched."""
    # exact sums, rounded by the exhaustive search
    for seed, (T, d, H) in enumerate([(3, 24, 5), (2, 40, 7), (4, 16, 3)]):
        x = synth.gelu_iid(T, d, seed=90 + seed)
        w = synth.down_weight(H, d, seed=90 + seed)
        a = o.decode(o.gelu_and_mul_sparse(x, BF16, Z95), BF16)
        wv = o.decode(w, BF16)
        exact = np.array([[float(sum(Fraction(float(a[r, k])) * Fraction(float(wv[h, k])) for k in range(d)))
                           for h in range(H)] for r in range(T)])
        y, f64, mag = o.gelu_and_mul_sparse_down(x, w, BF16, Z95, want_f64=True)
        assert np.array_equal(y, _nearest_bf16_bits(exact)), (T, d, H)
        assert np.all(np.abs(f64 - exact) <= d * 2.0 ** -52 * mag)
    # numpy's fp64 product and absolute sums
    T, d, H = 8, 512, 48
    for dt in (BF16, F16):
        x = synth.gelu_iid(T, d, seed=95, dtype=dt, gate_std=1.5)
        w = synth.down_weight(H, d, seed=95, dtype=dt)
        a = o.decode(o.gelu_and_mul_sparse(x, dt, Z95), dt)
        wv = o.decode(w, dt)
        y, f64, mag = o.gelu_and_mul_sparse_down(x, w, dt, Z95, want_f64=True)
        assert np.all(np.abs(f64 - a @ wv.T) <= 1e-12 * (np.abs(a) @ np.abs(wv).T))
        assert np.allclose(mag, np.abs(a) @ np.abs(wv).T, rtol=1e-12, atol=0)
        assert np.array_equal(y, o.encode(f64, dt))
    # one weight: y[:, h0] = a[:, k0] exactly, every other output 0 (H != d)
    T, d, H = 5, 96, 40
    x = synth.gelu_iid(T, d, seed=97, gate_std=1.0)
    a_bits = o.gelu_and_mul_sparse(x, BF16, 0.0)
    for h0, k0 in ((3, 71), (39, 0), (0, 95)):
        w = np.zeros((H, d), np.uint16)
        w[h0, k0] = 0x3F80                                     # 1.0
        y = o.gelu_and_mul_sparse_down(x, w, BF16, 0.0)
        # the same value (a -0 activation sums to +0)
        assert np.array_equal(o.decode(y[:, h0], BF16), o.decode(a_bits[:, k0], BF16))
        nz = o.decode(a_bits[:, k0], BF16) != 0
        assert nz.any() and np.array_equal(y[nz, h0], a_bits[nz, k0])
        rest = np.delete(y, h0, axis=1)
        assert np.all(o.decode(rest, BF16) == 0)
    # scaled permutation: y[r, h] = a[r, p(h)] * 2^e(h), exactly
    T, d = 6, 64
    x = synth.gelu_iid(T, d, seed=98)
    a = o.decode(o.gelu_and_mul_sparse(x, BF16, Z95), BF16)
    rng = _rng(98)
    perm, e = rng.permutation(d), rng.integers(-3, 4, d)
    wv = np.zeros((d, d))
    wv[np.arange(d), perm] = 2.0 ** e
    y = o.decode(o.gelu_and_mul_sparse_down(x, synth.to_bits(wv, BF16), BF16, Z95), BF16)
    assert np.array_equal(y, a[:, perm] * 2.0 ** e[None, :])
    # live rows only
    T, d, H = 7, 48, 9
    x = synth.gelu_iid(T, d, seed=99)
    w = synth.down_weight(H, d, seed=99)
    sentinel = np.full((T, H), synth.SENTINEL[BF16], np.uint16)
    full = o.gelu_and_mul_sparse_down(x, w, BF16, Z95)
    for live in (0, 3, 7, 12, -1):
        y = o.gelu_and_mul_sparse_down(x, w, BF16, Z95, live=live, out=sentinel)
        n = min(max(live, 0), T)
        assert np.array_equal(y[:n], full[:n]) and np.all(y[n:] == synth.SENTINEL[BF16])


ALL_PINS = [pin_decode, pin_encode_fp32, pin_encode_fp16, pin_encode_bf16,
            pin_roundtrip, pin_gelu, pin_silu, pin_row_stats,
            pin_gelu_sparse_composition, pin_gelu_sparse_invariants,
            pin_survival_fraction, pin_brute_force_1x8, pin_silu_bounded,
            pin_gelu_erf, pin_squared_relu, pin_gelu_and_mul, pin_squared_relu_bounded,
            pin_gelu_sparse_roundtrip, pin_down_projection]
