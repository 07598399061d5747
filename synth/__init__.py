"""Seeded synthetic inputs for the gated activations.

This module holds none of the method's arithmetic: it only draws random rows
and rounds them to the element type, so that the oracle and the GPU path can
be fed identical bits.  Both sides import it; neither side's arithmetic lives
here.

Random numbers come from a counter-based generator: value i of a stream is
the SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) applied to key + (i+1)*gamma.
Normals use the Box-Muller cosine branch on two uniforms; Student-t(3) is
Z / sqrt(chi2_3 / 3) with chi2_3 a sum of three squared normals.  The streams
run in a small C core (synth_core.c, glibc's log/cos/sqrt), not in numpy,
whose vectorised transcendentals can differ between host CPUs.

Every array returned is raw element bits: uint16 for bf16/fp16, uint32 for
fp32 (dtype codes 0 = fp32, 1 = fp16, 2 = bf16).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {"f32": F32, "f16": F16, "bf16": BF16}
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_THREADS = max(1, min(16, os.cpu_count() or 1))

# stream identifiers inside one seed
S_GATE, S_UP, S_OFFSET, S_KIND, S_WEIGHT = 1, 2, 3, 4, 5


def _core():
    global _CORE
    if _CORE is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.synth_normal.argtypes = [u64, i64, i64, ctypes.c_double, ctypes.c_double, vp, ctypes.c_int]
        lib.synth_raw64.argtypes = [u64, i64, i64, vp]
        lib.synth_uniform.argtypes = [u64, i64, i64, vp]
        lib.synth_normal_rows_bf16.argtypes = [u64, i64, i64, ctypes.c_double, ctypes.c_double,
                                               vp, i64, ctypes.c_int]
        for f in (lib.synth_normal, lib.synth_raw64, lib.synth_uniform, lib.synth_normal_rows_bf16):
            f.restype = None
        _CORE = lib
    return _CORE


_CORE = None


def _mix(x):
    x = (x ^ (x >> np.uint64(30))) * _M1
    x = (x ^ (x >> np.uint64(27))) * _M2
    return x ^ (x >> np.uint64(31))


def stream_key(seed: int, stream: int) -> np.uint64:
    """Key of one stream: the finaliser of (seed, stream) packed in 64 bits."""
    with np.errstate(over="ignore"):
        packed = np.array([(int(seed) & 0xFFFFFFFF) << 24 | (int(stream) & 0xFFFFFF)],
                          dtype=np.uint64)
        return _mix(packed * _GAMMA + _GAMMA)[0]


def raw64(key, start: int, n: int) -> np.ndarray:
    """Values start .. start+n-1 of the stream with this key (uint64)."""
    out = np.empty(n, np.uint64)
    _core().synth_raw64(int(key), start, n, out.ctypes.data)
    return out


def uniform(key, start: int, n: int) -> np.ndarray:
    """Uniforms in (0, 1]: the top 53 bits, plus one, times 2^-53."""
    out = np.empty(n, np.float64)
    _core().synth_uniform(int(key), start, n, out.ctypes.data)
    return out


def normal(key, start: int, n: int, scale: float = 1.0, shift: float = 0.0) -> np.ndarray:
    """shift + scale * standard normals; normal j uses stream values
    2(start+j) and 2(start+j)+1 (Box-Muller, cosine branch)."""
    out = np.empty(n, np.float64)
    _core().synth_normal(int(key), start, n, float(scale), float(shift), out.ctypes.data, _THREADS)
    return out


def student_t3(key, start: int, n: int) -> np.ndarray:
    """Student-t with 3 degrees of freedom; draw j uses normals 4(start+j)..+3."""
    z = normal(key, 4 * start, 4 * n).reshape(n, 4)
    chi2 = z[:, 1] ** 2 + z[:, 2] ** 2 + z[:, 3] ** 2
    return z[:, 0] / np.sqrt(chi2 / 3.0)


def to_bits(values: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 draws to the element type and return the bits.  (Input
    preparation only: fp32 and fp16 by numpy's casts, bf16 by ties-to-even on
    the fp32 bits.)"""
    v = np.asarray(values, dtype=np.float64)
    if dtype == F32:
        return v.astype(np.float32).view(np.uint32)
    if dtype == F16:
        return v.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
        u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
        return u.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype}")


def bits_to_float(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Element bits -> float32 view (for inspection and statistics in tests)."""
    b = np.asarray(bits)
    if dtype == F32:
        return b.view(np.float32)
    if dtype == F16:
        return b.view(np.float16).astype(np.float32)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Workload recipes.  Each returns element bits of shape [rows, 2d]: the gate
# in columns [0, d), up in [d, 2d).  "N(a, b)" means mean a, std b.
# ---------------------------------------------------------------------------

def normal_rows_into(out: np.ndarray, key, scale: float = 1.0, shift: float = 0.0,
                     dtype: int = BF16) -> None:
    """Fill the [rows, d] view `out` (row stride may exceed d) with element
    (r, i) = to_bits(shift + scale * normal(r * d + i)).  Same bits as the
    numpy route, done in one threaded pass for bf16."""
    rows, d = out.shape
    if dtype == BF16 and out.dtype == np.uint16 and out.strides[1] == 2:
        _core().synth_normal_rows_bf16(int(key), rows, d, float(scale), float(shift),
                                       out.ctypes.data, out.strides[0] // 2, _THREADS)
    else:
        out[...] = to_bits(normal(key, 0, rows * d, scale, shift).reshape(rows, d), dtype)


def _empty_rows(T: int, d: int, dtype: int) -> np.ndarray:
    return np.empty((T, 2 * d), np.uint32 if dtype == F32 else np.uint16)


def gelu_iid(T: int, d: int, seed: int = 0, dtype: int = BF16,
             gate_std: float = 1.0) -> np.ndarray:
    """Gate N(0, gate_std) and up N(0, 1), i.i.d.  T=4, d=2048, seed 0 is the
    small check case; gate_std=2 with seed T*1000 + d//1024 the large-row case."""
    x = _empty_rows(T, d, dtype)
    normal_rows_into(x[:, :d], stream_key(seed, S_GATE), scale=gate_std, dtype=dtype)
    normal_rows_into(x[:, d:], stream_key(seed, S_UP), dtype=dtype)
    return x


def gelu_offset_rows(T: int, d: int = 8192, seed: int = None,
                     dtype: int = BF16) -> np.ndarray:
    """Gate N(0,1) plus a per-row offset drawn from N(0, 0.5); up N(0,1).
    The token sweep uses seed = T."""
    seed = T if seed is None else seed
    off = 0.5 * normal(stream_key(seed, S_OFFSET), 0, T)
    g = normal(stream_key(seed, S_GATE), 0, T * d).reshape(T, d) + off[:, None]
    x = _empty_rows(T, d, dtype)
    x[:, :d] = to_bits(g, dtype)
    normal_rows_into(x[:, d:], stream_key(seed, S_UP), dtype=dtype)
    return x


def large_row_seed(T: int, d: int) -> int:
    return T * 1000 + d // 1024


def gelu_large(T: int, d: int, dtype: int = BF16) -> np.ndarray:
    """Large rows: gate N(0, 2), up N(0, 1), seed T*1000 + d//1024."""
    return gelu_iid(T, d, seed=large_row_seed(T, d), dtype=dtype, gate_std=2.0)


EDGE_KINDS = ("near_constant", "constant_drawn", "constant_zero",
              "constant_hundred", "student_t3")


def edge_rows(T: int, d: int, dtype: int, seed: int = None) -> np.ndarray:
    """Edge mix.  Row r takes kind EDGE_KINDS[r % 5]: N(100, 0.01) (variance
    cancellation), a constant drawn from N(0,1), the constant 0, the constant
    100, or Student-t(3) (heavy tails).  Up is N(0,1).  Seed d*1000 + T."""
    seed = d * 1000 + T if seed is None else seed
    kg = stream_key(seed, S_GATE)
    kc = stream_key(seed, S_OFFSET)
    g = np.empty((T, d), np.float64)
    for r in range(T):
        kind = EDGE_KINDS[r % len(EDGE_KINDS)]
        if kind == "near_constant":
            g[r] = 100.0 + 0.01 * normal(kg, r * d, d)
        elif kind == "constant_drawn":
            g[r] = normal(kc, r, 1)[0]
        elif kind == "constant_zero":
            g[r] = 0.0
        elif kind == "constant_hundred":
            g[r] = 100.0
        else:
            g[r] = student_t3(kg, r * d, d)
    x = _empty_rows(T, d, dtype)
    x[:, :d] = to_bits(g, dtype)
    normal_rows_into(x[:, d:], stream_key(seed, S_UP), dtype=dtype)
    return x


def moe_buffer(M: int = 16384, d: int = 768, seed: int = 7,
               dtype: int = BF16) -> np.ndarray:
    """Capture-sized MoE activation buffer [M, 2d], gate and up N(0, 1)."""
    return gelu_iid(M, d, seed=seed, dtype=dtype, gate_std=1.0)


def down_weight(H: int, d: int, seed: int = 0, dtype: int = BF16) -> np.ndarray:
    """Weights of the down projection that follows the activation: [H, d],
    one row of d weights per output feature, i.i.d. N(0, 1/d) (a linear
    layer's usual initial scale, so outputs stay of order one)."""
    w = np.empty((H, d), np.uint32 if dtype == F32 else np.uint16)
    normal_rows_into(w, stream_key(seed, S_WEIGHT), scale=1.0 / np.sqrt(d), dtype=dtype)
    return w


# Sentinel bits written to rows beyond the live count and to canary tails: a
# NaN payload that no kernel produces.
SENTINEL = {F32: np.uint32(0x7FA5A5A5), F16: np.uint16(0x7FA5), BF16: np.uint16(0x7FA5)}
