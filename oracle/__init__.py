"""ctypes/numpy front end of the C oracle.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product package.  Every function
mirrors one in oracle.c, which carries the citations of the method.

All bf16 arrays are numpy uint16 holding the bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _ptr(a, t):
    return a.ctypes.data_as(t)


class Oracle:
    """One loaded copy of the oracle library (tests may load mutants)."""

    def __init__(self, path=None):
        if path is None:
            path = _build.LIBRARY
            if not os.path.exists(path):
                _build.build()
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_rope_cossin.argtypes = [_f32p, _i64, _i64, _i64, _i64, _i64, _u16p, _u16p]
        lib.oracle_rope_cossin.restype = None
        lib.oracle_rope_angles_grid.restype = None
        lib.oracle_rope_angles_grid.argtypes = [_i64, _i64, _i64, _i64,
                                                ctypes.POINTER(ctypes.c_int32), ctypes.c_double,
                                                ctypes.POINTER(ctypes.c_int32), _f32p]
        lib.oracle_gemm_bf16.restype = None
        lib.oracle_gemm_bf16.argtypes = [_u16p, _i64, _i64, _i64, _u16p, _i64, _i64, _u16p, _i64]
        lib.oracle_gemm_geglu.restype = ctypes.c_int
        lib.oracle_gemm_geglu.argtypes = [_u16p, _i64, _i64, _i64, _u16p, _i64, _i64, _u16p, _i64]
        lib.oracle_rope_rows.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, _i64, _u16p]
        lib.oracle_rope_rows.restype = ctypes.c_int
        lib.oracle_rope_rotate_half.argtypes = [_u16p, _i64, _i64, _i64, _i64, _i64,
                                                _u16p, _u16p, _u16p]
        lib.oracle_rope_rotate_half.restype = ctypes.c_int
        lib.oracle_rope_rotate_half_exact.argtypes = [_f64p, _i64, _i64, _i64, _i64, _i64,
                                                      _f64p, _f64p, _f64p]
        lib.oracle_rope_rotate_half_exact.restype = None
        lib.oracle_gelu_exact.argtypes = [ctypes.c_double]
        lib.oracle_gelu_exact.restype = ctypes.c_double
        lib.oracle_gelu_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_gelu_bf16.restype = ctypes.c_uint16
        lib.oracle_gelu_and_mul.argtypes = [_u16p, _i64, _i64, _i64, _u16p, _i64]
        lib.oracle_gelu_and_mul.restype = None
        self.lib = lib

    # -- scalars -----------------------------------------------------------
    def bf16_to_double(self, b):
        return self.lib.oracle_bf16_to_double(int(b))

    def double_to_bf16(self, v, sticky=0):
        return self.lib.oracle_double_to_bf16(float(v), int(sticky))

    def gelu_exact(self, x):
        return self.lib.oracle_gelu_exact(float(x))

    def gelu_bf16(self, g):
        return self.lib.oracle_gelu_bf16(int(g))

    def gelu_table(self):
        """rne_bf16(GELU(x)) for all 65536 bf16 bit patterns x."""
        return np.array([self.lib.oracle_gelu_bf16(i) for i in range(65536)], dtype=np.uint16)

    # -- Cos/sin tables -------------------------------------------------
    def rope_cossin(self, freqs):
        """freqs: float32 (S, B, 1, R) array (any strides with unit last stride).

        Returns (cos, sin), each uint16 (B*S, R), row b*S + s.
        """
        freqs = np.asarray(freqs)
        assert freqs.dtype == np.float32 and freqs.ndim == 4 and freqs.shape[2] == 1
        S, B, _, R = freqs.shape
        if freqs.strides[3] != 4:
            freqs = np.ascontiguousarray(freqs)
        ss, sb = freqs.strides[0] // 4, freqs.strides[1] // 4
        cos = np.empty((B * S, R), np.uint16)
        sin = np.empty((B * S, R), np.uint16)
        base = freqs.ctypes.data_as(_f32p)
        self.lib.oracle_rope_cossin(base, S, B, R, ss, sb, _ptr(cos, _u16p), _ptr(sin, _u16p))
        return cos, sin

    def rope_angles_grid(self, B, grid, dims, theta, t_offset=None):
        """fp32 angles (S, B, 1, R) of a (T, Hg, Wg) token grid with axis
        column counts `dims` (3 even ints); t_offset: B ints or None."""
        T, Hg, Wg = (int(v) for v in grid)
        d = np.ascontiguousarray(dims, np.int32)
        assert d.shape == (3,) and (d % 2 == 0).all()
        S, R = T * Hg * Wg, int(d.sum())
        out = np.empty((S, B, 1, R), np.float32)
        off = None
        if t_offset is not None:
            off = np.ascontiguousarray(t_offset, np.int32)
            assert off.shape == (B,)
        self.lib.oracle_rope_angles_grid(
            B, T, Hg, Wg, _ptr(d, ctypes.POINTER(ctypes.c_int32)), float(theta),
            None if off is None else _ptr(off, ctypes.POINTER(ctypes.c_int32)),
            _ptr(out, _f32p))
        return out

    def rope_cossin_grid(self, B, grid, dims, theta, t_offset=None):
        """The (B*S, R) cos/sin tables of the grid's angles."""
        return self.rope_cossin(self.rope_angles_grid(B, grid, dims, theta, t_offset))

    # -- Gate_up projection and GEGLU on it -----------------------------
    def gemm_bf16(self, x, w):
        """x: uint16 (M, K), w: uint16 (N, K).  Returns rne_bf16(x w^T), (M, N)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        (M, K), (N, K2) = x.shape, w.shape
        assert K == K2
        out = np.empty((M, N), np.uint16)
        self.lib.oracle_gemm_bf16(_ptr(x, _u16p), M, K, K, _ptr(w, _u16p), N, K,
                                  _ptr(out, _u16p), N)
        return out

    def gemm_geglu(self, x, w):
        """x: uint16 (M, K), w: uint16 (2H, K), gate rows first.  Returns (M, H)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        (M, K), (N, K2) = x.shape, w.shape
        assert K == K2 and N % 2 == 0
        out = np.empty((M, N // 2), np.uint16)
        rc = self.lib.oracle_gemm_geglu(_ptr(x, _u16p), M, K, K, _ptr(w, _u16p), N // 2, K,
                                        _ptr(out, _u16p), N // 2)
        assert rc == 0
        return out

    # -- Rotate-half ------------------------------------------------
    def rope_rotate_half(self, x, cos, sin):
        """x: uint16 (B, S, H, D); cos/sin: uint16 (B*S, R).  Returns out (B, S, H, D)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        cos = np.ascontiguousarray(cos, dtype=np.uint16)
        sin = np.ascontiguousarray(sin, dtype=np.uint16)
        B, S, H, D = x.shape
        R = cos.shape[1]
        assert cos.shape == (B * S, R) and sin.shape == (B * S, R)
        out = np.empty_like(x)
        rc = self.lib.oracle_rope_rotate_half(_ptr(x, _u16p), B, S, H, D, R, _ptr(cos, _u16p),
                                              _ptr(sin, _u16p), _ptr(out, _u16p))
        if rc != 0:
            raise ValueError("oracle_rope_rotate_half: bad shape")
        return out

    def rope_rows(self, x_rows, cos_rows, sin_rows):
        """x_rows: uint16 (n, D); cos_rows/sin_rows: uint16 (n, R) (row i rotates with row i)."""
        x_rows = np.ascontiguousarray(x_rows, dtype=np.uint16)
        cos_rows = np.ascontiguousarray(cos_rows, dtype=np.uint16)
        sin_rows = np.ascontiguousarray(sin_rows, dtype=np.uint16)
        n, D = x_rows.shape
        R = cos_rows.shape[1]
        assert cos_rows.shape == (n, R) and sin_rows.shape == (n, R)
        out = np.empty_like(x_rows)
        rc = self.lib.oracle_rope_rows(_ptr(x_rows, _u16p), _ptr(cos_rows, _u16p),
                                       _ptr(sin_rows, _u16p), n, D, R, _ptr(out, _u16p))
        if rc != 0:
            raise ValueError("oracle_rope_rows: bad shape")
        return out

    def rope_rotate_half_exact(self, x, cos, sin):
        """Exact-arithmetic policy: float64 x (B,S,H,D), float64 cos/sin (B*S, R)."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        cos = np.ascontiguousarray(cos, dtype=np.float64)
        sin = np.ascontiguousarray(sin, dtype=np.float64)
        B, S, H, D = x.shape
        R = cos.shape[1]
        out = np.empty_like(x)
        self.lib.oracle_rope_rotate_half_exact(_ptr(x, _f64p), B, S, H, D, R, _ptr(cos, _f64p),
                                               _ptr(sin, _f64p), _ptr(out, _f64p))
        return out

    # -- GEGLU ------------------------------------------------------
    def gelu_and_mul(self, inp):
        """inp: uint16 (rows, 2*hidden), gate first then up.  Returns (rows, hidden)."""
        inp = np.ascontiguousarray(inp, dtype=np.uint16)
        rows, two_h = inp.shape
        assert two_h % 2 == 0
        hidden = two_h // 2
        out = np.empty((rows, hidden), np.uint16)
        self.lib.oracle_gelu_and_mul(_ptr(inp, _u16p), rows, hidden, two_h, _ptr(out, _u16p),
                                     hidden)
        return out


_default = None


def get():
    """The oracle built from oracle/oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
