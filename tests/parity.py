"""Comparison of GPU output with the fp64 oracle, and device plumbing for tests.

Tolerance: each element of a live row must be within max(2 ulp of the output
type at the oracle's value, 1e-3) of the oracle.  For gelu_and_mul_sparse the
only elements allowed to miss are those whose gate lies within 1e-4 * std of
the cutoff (std and cutoff from the oracle), where fp32 and fp64 may take
opposite sides of the threshold; they must number fewer than 1e-4 of all
elements.  Rows beyond the live count and a canary tail after every output
buffer must keep their sentinel bits exactly.
"""
import numpy as np
import torch

import synth

F32, F16, BF16 = synth.F32, synth.F16, synth.BF16
TORCH_DTYPE = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}
INT_VIEW = {F32: torch.int32, F16: torch.int16, BF16: torch.int16}
NP_BITS = {F32: np.uint32, F16: np.uint16, BF16: np.uint16}
MANT_BITS = {F32: 23, F16: 10, BF16: 7}
EMIN = {F32: -126, F16: -14, BF16: -126}
CANARY = 4096
Z95 = float(np.float32(1.6448536))
Z99 = float(np.float32(2.3263479))


def decode(bits, dtype):
    b = np.asarray(bits)
    if dtype == F32:
        return b.view(np.float32).astype(np.float64)
    if dtype == F16:
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def ulp(y, dtype):
    """Spacing of the output type at |y| (the subnormal spacing below emin)."""
    a = np.abs(y)
    _, e = np.frexp(a)
    e = np.maximum(e - 1, EMIN[dtype])
    return np.ldexp(1.0, e - MANT_BITS[dtype])


def to_device(bits, dtype, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(
        np.int32 if dtype == F32 else np.int16)).to(device)
    return t.view(TORCH_DTYPE[dtype])


def sentinel_buffer(rows, d, dtype, device="cuda"):
    """A [rows, d] output view whose storage carries a canary tail; every
    element (and the tail) starts as the sentinel bit pattern."""
    s = int(synth.SENTINEL[dtype])
    if s >= 1 << (31 if dtype == F32 else 15):
        s -= 1 << (32 if dtype == F32 else 16)
    buf = torch.full((rows * d + CANARY,), s, dtype=INT_VIEW[dtype], device=device)
    return buf, buf[: rows * d].view(rows, d).view(TORCH_DTYPE[dtype])


def bits_of(t, dtype):
    return t.contiguous().view(INT_VIEW[dtype]).cpu().numpy().view(NP_BITS[dtype])


def check_canary(buf, rows, d, dtype):
    tail = bits_of(buf[rows * d:], dtype)
    assert np.all(tail == synth.SENTINEL[dtype]), "canary tail after the output was overwritten"


def compare(gpu_bits, ora_bits, dtype, gate=None, stats=None, label=""):
    """Element-wise check of live rows.  gate / stats (mean, std, cutoff per
    row, from the oracle) enable the gelu exemption band.  Returns a summary."""
    g = decode(gpu_bits, dtype)
    o = decode(ora_bits, dtype)
    assert not np.isnan(g[~np.isnan(o)]).any(), f"{label}: NaN in GPU output"
    same_inf = np.isinf(g) & np.isinf(o) & (np.sign(g) == np.sign(o))
    err = np.where(same_inf, 0.0, np.abs(g - o))
    tol = np.maximum(2.0 * ulp(o, dtype), 1e-3)
    bad = err > tol
    n_bad = int(bad.sum())
    out = {"elements": int(g.size), "max_abs_err": float(err.max()) if err.size else 0.0,
           "max_err_ulp": float((err / ulp(o, dtype)).max()) if err.size else 0.0,
           "bitexact_frac": float((np.asarray(gpu_bits) == np.asarray(ora_bits)).mean()) if err.size else 1.0,
           "n_out_of_tol": n_bad, "n_exempt": 0}
    if stats is not None:
        cut = stats[2][:, None]
        std = stats[1][:, None]
        dist = np.abs(gate - cut)
        band = dist < 1e-4 * std
        if (bad & ~band).any():
            idx = np.argwhere(bad & ~band)[:5]
            detail = "; ".join(f"row {r} col {c}: gate={gate[r, c]!r} cut={cut[r, 0]!r} "
                               f"oracle={o[r, c]!r} gpu={g[r, c]!r}" for r, c in idx)
            raise AssertionError(f"{label}: {int((bad & ~band).sum())} elements out of tolerance "
                                 f"outside the exemption band: {detail}")
        out["n_exempt"] = n_bad
        assert n_bad < 1e-4 * g.size or n_bad == 0, f"{label}: {n_bad} exempt elements >= 1e-4 of all"
        # Mask diagnostic, outside a band widened to the resolution at which
        # fp32 can hold the cutoff: an element the oracle masks must come back
        # as exactly +-0 (0 * up), and one the oracle passes must not be zero
        # unless its true value underflows the output type.
        wide = np.maximum(1e-4 * std, 4.0 * np.abs(cut) * 2.0 ** -23)
        passes = gate > cut
        min_normal = 2.0 ** EMIN[dtype]
        flip = (dist >= wide) & ((~passes & (g != 0)) |
                                 (passes & (g == 0) & (np.abs(o) >= min_normal)))
        out["mask_mismatch_outside_band"] = int(flip.sum())
        if flip.any():
            idx = np.argwhere(flip)[:5]
            detail = "; ".join(f"row {r} col {c}: gate={gate[r, c]!r} cut={cut[r, 0]!r} "
                               f"std={std[r, 0]!r} oracle={o[r, c]!r} gpu={g[r, c]!r}"
                               for r, c in idx)
            raise AssertionError(f"{label}: {int(flip.sum())} zero-mask mismatches outside the band: {detail}")
    else:
        assert n_bad == 0, f"{label}: {n_bad} elements out of tolerance (max err {out['max_abs_err']:.3g})"
    return out
