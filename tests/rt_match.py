"""Matching of the GPU's round-trip form against the oracle (bf16 / fp16).

Where the GPU's fp32 row statistics can round to a different element-type
value than the oracle's exact ones, several cutoffs are legitimate; see
tests/test_gpu_roundtrip.py for the bounds used and why.
"""
import itertools

import numpy as np

from parity import decode, ulp

EPS32 = 2.0 ** -24
RED_DEPTH = 128   # bound on the sequential depth of the GPU's fp32 row reductions
MAX_CANDIDATES = 64  # rows whose cutoff lies near zero (fp16 spacing is fine there) need up to ~30


def _rn(o, v, dtype):
    """Round-to-nearest-even of doubles into the element type, as doubles."""
    return decode(o.encode(np.atleast_1d(np.asarray(v, np.float64)), dtype), dtype)


def _next_up16(bits):
    """Next 16-bit float pattern upwards, with -0 folded into +0."""
    b = int(bits)
    if b == 0x8001:
        return 0x0000
    return b + 1 if b < 0x8000 else b - 1


def cut_candidates(o, gate, dtype, z):
    """Per row, the element-type cutoffs the GPU can reach (bounds in
    tests/test_gpu_roundtrip.py); None for a row with more than MAX_CANDIDATES."""
    g = np.asarray(gate, np.float64)
    mu = g.mean(axis=1)
    sigma = np.sqrt(((g - mu[:, None]) ** 2).mean(axis=1))
    abs_mean = np.abs(g).mean(axis=1)
    dm = RED_DEPTH * EPS32 * abs_mean + 2 * EPS32 * np.abs(mu)
    rel_v = (RED_DEPTH + 4) * EPS32
    s_lo = np.sqrt(np.maximum(sigma ** 2 * (1 - rel_v), 0.0)) * (1 - EPS32)
    s_hi = np.sqrt((sigma ** 2 + dm ** 2) * (1 + rel_v)) * (1 + EPS32)
    z_r = _rn(o, float(np.float32(z)), dtype)[0]
    out = []
    for r in range(g.shape[0]):
        corners = []
        for m, s in itertools.product((mu[r] - dm[r], mu[r] + dm[r]), (s_lo[r], s_hi[r])):
            zs = _rn(o, z_r * _rn(o, s, dtype)[0], dtype)[0]
            corners.append(_rn(o, _rn(o, m, dtype)[0] + zs, dtype)[0])
        lo, hi = min(corners) + 0.0, max(corners) + 0.0   # -0 -> +0
        bits = int(o.encode(np.array([lo]), dtype)[0])
        stop = int(o.encode(np.array([hi]), dtype)[0])
        cands = [lo]
        while bits != stop and len(cands) <= MAX_CANDIDATES:
            bits = _next_up16(bits)
            cands.append(float(decode(np.array([bits], np.uint16), dtype)[0]))
        out.append(cands if len(cands) <= MAX_CANDIDATES else None)
    return out


def rows_match(got, ref, dtype):
    """Per row: every element within 3 ulp of the oracle (bound in tests/test_gpu_roundtrip.py)."""
    g, o = decode(got, dtype), decode(ref, dtype)
    same_inf = np.isinf(g) & np.isinf(o) & (np.sign(g) == np.sign(o))
    err = np.where(same_inf, 0.0, np.abs(g - o))
    err = np.where(np.isnan(err), np.inf, err)
    return (err <= 3.0 * ulp(o, dtype)).all(axis=1)
