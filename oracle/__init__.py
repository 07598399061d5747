"""ctypes front end of the fp64 CPU oracle (oracle/ga_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  Arrays cross the
boundary as raw element bits: uint16 for bf16/fp16, uint32 for fp32, so the
oracle and the GPU path see identical input bits.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, F16, BF16 = 0, 1, 2
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}
BITS_DTYPE = {F32: np.uint32, F16: np.uint16, BF16: np.uint16}

_lib = None


def _load(path=None):
    lib = ctypes.CDLL(path or _build.LIB)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.gao_decode.restype = dbl
    lib.gao_decode.argtypes = [ctypes.c_uint32, ctypes.c_int]
    lib.gao_encode_rne.restype = ctypes.c_uint32
    lib.gao_encode_rne.argtypes = [dbl, ctypes.c_int]
    lib.gao_gelu_tanh.restype = dbl
    lib.gao_gelu_tanh.argtypes = [dbl]
    lib.gao_silu.restype = dbl
    lib.gao_silu.argtypes = [dbl]
    lib.gao_row_stats.restype = None
    lib.gao_row_stats.argtypes = [vp, i64, vp, vp]
    lib.gao_gelu_and_mul_sparse.restype = ctypes.c_int
    lib.gao_gelu_and_mul_sparse.argtypes = [vp, vp, i64, i64, ctypes.c_int,
                                            ctypes.c_float, i64, vp, vp, vp, vp]
    lib.gao_silu_and_mul_bounded.restype = ctypes.c_int
    lib.gao_silu_and_mul_bounded.argtypes = [vp, vp, i64, i64, ctypes.c_int,
                                             i64, vp]
    for name in ("gao_decode_array", "gao_encode_array"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [vp, i64, ctypes.c_int, vp]
    lib.gao_gelu_and_mul_sparse_rt.restype = ctypes.c_int
    lib.gao_gelu_and_mul_sparse_rt.argtypes = [vp, vp, i64, i64, ctypes.c_int, ctypes.c_float, i64,
                                               vp, vp, vp, vp]
    lib.gao_gelu_and_mul.restype = ctypes.c_int
    lib.gao_gelu_and_mul.argtypes = [vp, vp, i64, i64, ctypes.c_int, ctypes.c_int, i64, vp]
    lib.gao_gelu_and_mul_sparse_down.restype = ctypes.c_int
    lib.gao_gelu_and_mul_sparse_down.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                                 i64, vp, vp]
    lib.gao_squared_relu_bounded.restype = ctypes.c_int
    lib.gao_squared_relu_bounded.argtypes = [vp, vp, i64, i64, ctypes.c_int, i64, vp]
    for name in ("gao_gelu_tanh_array", "gao_silu_array", "gao_gelu_erf_array", "gao_squared_relu_array"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [vp, i64, vp]
    return lib


class Oracle:
    """One loaded copy of the oracle library (the default one, or a mutant
    built from an edited copy of the source for the planted-mistake tests)."""

    def __init__(self, path=None):
        self.lib = _load(path)

    # -- codec ------------------------------------------------------------
    def decode(self, bits, dtype):
        bits = np.ascontiguousarray(bits, dtype=BITS_DTYPE[dtype])
        out = np.empty(bits.shape, np.float64)
        self.lib.gao_decode_array(bits.ctypes.data, bits.size, dtype, out.ctypes.data)
        return out

    def encode(self, values, dtype):
        v = np.ascontiguousarray(values, dtype=np.float64)
        out = np.empty(v.shape, BITS_DTYPE[dtype])
        self.lib.gao_encode_array(v.ctypes.data, v.size, dtype, out.ctypes.data)
        return out

    # -- elementwise steps ---------------------------------------------------
    def gelu_tanh(self, s):
        s = np.ascontiguousarray(s, dtype=np.float64)
        out = np.empty(s.shape, np.float64)
        self.lib.gao_gelu_tanh_array(s.ctypes.data, s.size, out.ctypes.data)
        return out

    def _map(self, fn, x):
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, np.float64)
        fn(x.ctypes.data, x.size, out.ctypes.data)
        return out

    def silu(self, x):
        return self._map(self.lib.gao_silu_array, x)

    def gelu_erf(self, x):
        return self._map(self.lib.gao_gelu_erf_array, x)

    def squared_relu(self, x):
        return self._map(self.lib.gao_squared_relu_array, x)

    def row_stats(self, g):
        g = np.ascontiguousarray(g, dtype=np.float64)
        mean, std = ctypes.c_double(), ctypes.c_double()
        self.lib.gao_row_stats(g.ctypes.data, g.size, ctypes.byref(mean), ctypes.byref(std))
        return mean.value, std.value

    # -- whole ops -------------------------------------------------------------
    def gelu_and_mul_sparse(self, x_bits, dtype, z, live=None, out=None,
                            want_f64=False, want_stats=False):
        """x_bits: [T, 2d] element bits.  Returns out bits [T, d] (rows >= live
        keep the contents of `out` if given, else zeros), plus the unrounded
        product and (mean, std, cutoff) per row when asked."""
        x = np.ascontiguousarray(x_bits, dtype=BITS_DTYPE[dtype])
        T, two_d = x.shape
        d = two_d // 2
        assert two_d == 2 * d and d >= 1
        live = T if live is None else int(live)
        y = np.zeros((T, d), BITS_DTYPE[dtype]) if out is None else np.array(out, copy=True)
        f64 = np.full((T, d), np.nan) if want_f64 else None
        stats = np.full((3, T), np.nan) if want_stats else None
        p = lambda a: None if a is None else a.ctypes.data  # noqa: E731
        rc = self.lib.gao_gelu_and_mul_sparse(
            x.ctypes.data, y.ctypes.data, T, d, dtype, float(z), live, p(f64),
            None if stats is None else stats[0].ctypes.data,
            None if stats is None else stats[1].ctypes.data,
            None if stats is None else stats[2].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        res = [y]
        if want_f64:
            res.append(f64)
        if want_stats:
            res.append(stats)
        return res[0] if len(res) == 1 else tuple(res)

    def gelu_and_mul_sparse_rt(self, x_bits, dtype, z, live=None, out=None, cut=None):
        """Round-trip form (intermediates rounded to the element type).
        Returns (out bits, stats[3, T]) with stats = exact mean, exact std,
        rounded cutoff used; `cut` (per-row, element-type values) overrides
        the computed cutoffs."""
        x = np.ascontiguousarray(x_bits, dtype=BITS_DTYPE[dtype])
        T, two_d = x.shape
        d = two_d // 2
        assert two_d == 2 * d and d >= 1
        live = T if live is None else int(live)
        y = np.zeros((T, d), BITS_DTYPE[dtype]) if out is None else np.array(out, copy=True)
        stats = np.full((3, T), np.nan)
        cut_arr = None if cut is None else np.ascontiguousarray(cut, dtype=np.float64)
        rc = self.lib.gao_gelu_and_mul_sparse_rt(
            x.ctypes.data, y.ctypes.data, T, d, dtype, float(z), live,
            None if cut_arr is None else cut_arr.ctypes.data,
            stats[0].ctypes.data, stats[1].ctypes.data, stats[2].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, stats

    def silu_and_mul_bounded(self, x_bits, dtype, live, out=None, want_f64=False):
        x = np.ascontiguousarray(x_bits, dtype=BITS_DTYPE[dtype])
        M, two_d = x.shape
        d = two_d // 2
        assert two_d == 2 * d and d >= 1
        y = np.zeros((M, d), BITS_DTYPE[dtype]) if out is None else np.array(out, copy=True)
        f64 = np.full((M, d), np.nan) if want_f64 else None
        rc = self.lib.gao_silu_and_mul_bounded(
            x.ctypes.data, y.ctypes.data, M, d, dtype, int(live),
            None if f64 is None else f64.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return (y, f64) if want_f64 else y

    def gelu_and_mul(self, x_bits, dtype, approximate, live=None, out=None, want_f64=False):
        """Non-sparse GELU-and-multiply; approximate: True = tanh form,
        False = exact erf form."""
        x = np.ascontiguousarray(x_bits, dtype=BITS_DTYPE[dtype])
        T, two_d = x.shape
        d = two_d // 2
        assert two_d == 2 * d and d >= 1
        live = T if live is None else int(live)
        y = np.zeros((T, d), BITS_DTYPE[dtype]) if out is None else np.array(out, copy=True)
        f64 = np.full((T, d), np.nan) if want_f64 else None
        rc = self.lib.gao_gelu_and_mul(x.ctypes.data, y.ctypes.data, T, d, dtype, int(bool(approximate)),
                                       live, None if f64 is None else f64.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return (y, f64) if want_f64 else y

    def gelu_and_mul_sparse_down(self, x_bits, w_bits, dtype, z, live=None, out=None, want_f64=False):
        """Sparse GELU-and-multiply of x[T, 2d], then the down projection
        y[T, H] = a . w^T with w[H, d] (rows of weights per output feature).
        Returns y bits (rows >= live keep `out`'s contents if given, else
        zeros), plus (unrounded sums, sums of |a w|) when want_f64."""
        x = np.ascontiguousarray(x_bits, dtype=BITS_DTYPE[dtype])
        w = np.ascontiguousarray(w_bits, dtype=BITS_DTYPE[dtype])
        T, two_d = x.shape
        d = two_d // 2
        H = w.shape[0]
        assert two_d == 2 * d and d >= 1 and w.shape == (H, d) and H >= 1
        live = T if live is None else int(live)
        y = np.zeros((T, H), BITS_DTYPE[dtype]) if out is None else np.array(out, copy=True)
        assert y.shape == (T, H)
        f64 = np.full((T, H), np.nan) if want_f64 else None
        mag = np.full((T, H), np.nan) if want_f64 else None
        rc = self.lib.gao_gelu_and_mul_sparse_down(
            x.ctypes.data, w.ctypes.data, y.ctypes.data, T, d, H, dtype, float(z), live,
            None if f64 is None else f64.ctypes.data, None if mag is None else mag.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return (y, f64, mag) if want_f64 else y

    def squared_relu_bounded(self, x_bits, dtype, live, out=None, want_f64=False):
        """Bounded squared ReLU of x[M, d] (not gated)."""
        x = np.ascontiguousarray(x_bits, dtype=BITS_DTYPE[dtype])
        M, d = x.shape
        y = np.zeros((M, d), BITS_DTYPE[dtype]) if out is None else np.array(out, copy=True)
        f64 = np.full((M, d), np.nan) if want_f64 else None
        rc = self.lib.gao_squared_relu_bounded(x.ctypes.data, y.ctypes.data, M, d, dtype, int(live),
                                               None if f64 is None else f64.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return (y, f64) if want_f64 else y


def get():
    """The default oracle, building it first if no library is there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = Oracle()
    return _lib
