"""CPU oracle for block-quantized weight GEMV (Q4_0 / Q8_0) — test infrastructure.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``quantized_weight_gemv_amd``) never imports it, and it imports nothing from
the product: it parses the packed bytes with its own code (``oracle.c``).

The arithmetic lives in ``oracle.c`` (plain fp64 C, built with gcc); this module
only loads it and marshals numpy arrays.  Each wrapper names the definition it
follows; the definitions themselves are stated in ``oracle.c``'s header.

Parity pins (tests/test_oracle.py): binary16 codec against numpy's, hand-derived
worked blocks (tests/golden/), brute-force nearest-code search, exact rational
GEMV on tiny shapes, closed forms (one-hot, zero, all-ones), invariants and
planted-mistake builds.  Every function here is pinned; none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q4_0 = 0
Q8_0 = 1
Q2W = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(plant: str | None = None, out: str | None = None) -> str:
    """Compile oracle.c with gcc (fp64, no FMA contraction, OpenMP over rows).

    ``plant`` builds a deliberately broken copy (an ``ORC_PLANT_*`` macro of
    oracle.c) used by the tests to show that the pins catch plausible mistakes;
    the product never sees such a build.
    """
    out = out or _LIB
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-o", out]
    if plant:
        cmd += [f"-DORC_PLANT_{plant.upper()}=1"]
    cmd += [_SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """ctypes view of one build of oracle.c."""

    def __init__(self, path: str = _LIB):
        if not os.path.exists(path):
            if path != _LIB:
                raise FileNotFoundError(path)
            build()
        elif path == _LIB and os.path.getmtime(_SRC) > os.path.getmtime(_LIB):
            build()   # the source changed since the library was built
        L = ctypes.CDLL(path)
        self._L = L
        u8p, u16p, f32p, f64p = (ctypes.POINTER(t) for t in
                                 (ctypes.c_uint8, ctypes.c_uint16, ctypes.c_float, ctypes.c_double))
        i64, sz = ctypes.c_int64, ctypes.c_size_t
        L.orc_half_to_double.restype = ctypes.c_double
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_double_to_half.restype = ctypes.c_uint16
        L.orc_double_to_half.argtypes = [ctypes.c_double]
        L.orc_float_to_half.restype = ctypes.c_uint16
        L.orc_float_to_half.argtypes = [ctypes.c_float]
        L.orc_packed_bytes.restype = sz
        L.orc_packed_bytes.argtypes = [ctypes.c_int, i64, i64]
        L.orc_quantize.restype = ctypes.c_int
        L.orc_quantize.argtypes = [ctypes.c_int, f32p, i64, i64, u8p, sz]
        for name, outp in (("orc_dequant_f64", f64p), ("orc_dequant_f32", f32p), ("orc_dequant_f16", u16p)):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [ctypes.c_int, u8p, i64, i64, outp]
        L.orc_gemv.restype = None
        L.orc_gemv.argtypes = [ctypes.c_int, u8p, i64, i64, u16p, i64, f64p, f64p]
        L.orc_gemv_rows.restype = None
        L.orc_gemv_rows.argtypes = [ctypes.c_int, u8p, i64, i64, u16p, i64,
                                    ctypes.POINTER(ctypes.c_int64), i64, f64p, f64p]
        L.orc_moe.restype = None
        L.orc_moe.argtypes = [ctypes.c_int, u8p, i64, ctypes.POINTER(ctypes.c_int32), i64,
                              u16p, i64, i64, f64p, f64p]
        L.orc_floats_to_half.restype = None
        L.orc_floats_to_half.argtypes = [f32p, i64, u16p]
        L.orc_silu.restype = ctypes.c_double
        L.orc_silu.argtypes = [ctypes.c_double]
        L.orc_swiglu.restype = None
        L.orc_swiglu.argtypes = [f64p, f64p, i64, f64p]
        i8p = ctypes.POINTER(ctypes.c_int8)
        L.orc_quantize_act8.restype = None
        L.orc_quantize_act8.argtypes = [u16p, i64, i64, i8p, f32p]
        L.orc_gemv_q8act.restype = None
        L.orc_gemv_q8act.argtypes = [ctypes.c_int, u8p, i64, i64, i8p, f32p, i64, f64p, f64p]
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_max_threads.argtypes = []

    def set_threads(self, n: int):
        """OpenMP threads of the row loops (no change to any result)."""
        self._L.orc_set_threads(int(n))

    def max_threads(self) -> int:
        return int(self._L.orc_max_threads())

    # -- helpers ---------------------------------------------------------
    @staticmethod
    def _p(a: np.ndarray, ctype):
        assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
        return a.ctypes.data_as(ctypes.POINTER(ctype))

    @staticmethod
    def _x16(x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x)
        if x.dtype == np.float16:
            x = x.view(np.uint16)
        assert x.dtype == np.uint16
        return x

    # -- binary16 codec --------------------------------------------------
    def half_to_double(self, h: int) -> float:
        return self._L.orc_half_to_double(int(h))

    def double_to_half(self, v: float) -> int:
        return int(self._L.orc_double_to_half(float(v)))

    def float_to_half(self, v) -> int:
        return int(self._L.orc_float_to_half(float(np.float32(v))))

    # -- format ----------------------------------------------------------
    def packed_bytes(self, fmt: int, N: int, K: int) -> int:
        return int(self._L.orc_packed_bytes(fmt, N, K))

    def quantize(self, fmt: int, w: np.ndarray) -> np.ndarray:
        """Quantize + pack fp32 [N][K] weights (block rule in oracle.c)."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        N, K = w.shape
        nbytes = self.packed_bytes(fmt, N, K)
        if nbytes == 0:
            raise ValueError("bad shape")
        out = np.empty(nbytes, dtype=np.uint8)
        rc = self._L.orc_quantize(fmt, self._p(w, ctypes.c_float), N, K,
                                  self._p(out, ctypes.c_uint8), nbytes)
        if rc != 0:
            raise ValueError(f"oracle quantizer rejected the weights (code {rc})")
        return out

    def dequant(self, fmt: int, packed: np.ndarray, N: int, K: int, out: str = "f64") -> np.ndarray:
        """Exact dequantized weights: f64 / f32 values, or f16 (returned as float16)."""
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        assert packed.size >= self.packed_bytes(fmt, N, K)
        if out == "f64":
            r = np.empty((N, K), np.float64)
            self._L.orc_dequant_f64(fmt, self._p(packed, ctypes.c_uint8), N, K, self._p(r, ctypes.c_double))
        elif out == "f32":
            r = np.empty((N, K), np.float32)
            self._L.orc_dequant_f32(fmt, self._p(packed, ctypes.c_uint8), N, K, self._p(r, ctypes.c_float))
        elif out == "f16":
            r = np.empty((N, K), np.uint16)
            self._L.orc_dequant_f16(fmt, self._p(packed, ctypes.c_uint8), N, K, self._p(r, ctypes.c_uint16))
            r = r.view(np.float16)
        else:
            raise ValueError(out)
        return r

    def gemv(self, fmt: int, packed: np.ndarray, N: int, K: int, x: np.ndarray):
        """(y, s): y[m][n] = sum_k w[n][k] x[m][k] in fp64, s = sum |w x|."""
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        x = self._x16(x)
        M = x.shape[0]
        assert x.shape == (M, K)
        y = np.empty((M, N), np.float64)
        s = np.empty((M, N), np.float64)
        self._L.orc_gemv(fmt, self._p(packed, ctypes.c_uint8), N, K, self._p(x, ctypes.c_uint16), M,
                         self._p(y, ctypes.c_double), self._p(s, ctypes.c_double))
        return y, s

    def gemv_rows(self, fmt: int, packed: np.ndarray, N: int, K: int, x: np.ndarray, rows):
        """The GEMV definition on selected rows: (y, s) of shape [M][len(rows)]."""
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        x = self._x16(x)
        M = x.shape[0]
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < N)
        y = np.empty((M, rows.size), np.float64)
        s = np.empty((M, rows.size), np.float64)
        self._L.orc_gemv_rows(fmt, self._p(packed, ctypes.c_uint8), N, K, self._p(x, ctypes.c_uint16), M,
                              self._p(rows, ctypes.c_int64), rows.size,
                              self._p(y, ctypes.c_double), self._p(s, ctypes.c_double))
        return y, s

    def moe(self, fmt: int, pool: np.ndarray, P: int, idx: np.ndarray, x: np.ndarray, N: int, K: int):
        """(y, s) of shape [E][N]: expert e = pool matrix idx[e] times token x[e]."""
        pool = np.ascontiguousarray(pool, dtype=np.uint8)
        assert pool.size >= P * self.packed_bytes(fmt, N, K)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        x = self._x16(x)
        E = idx.size
        assert x.shape == (E, K)
        y = np.empty((E, N), np.float64)
        s = np.empty((E, N), np.float64)
        self._L.orc_moe(fmt, self._p(pool, ctypes.c_uint8), P, self._p(idx, ctypes.c_int32), E,
                        self._p(x, ctypes.c_uint16), N, K, self._p(y, ctypes.c_double),
                        self._p(s, ctypes.c_double))
        return y, s

    def prefill(self, packed: np.ndarray, N: int, K: int, X: np.ndarray):
        """Q4_0 prefill GEMM: the GEMV definition over M token rows (fp64, exact weights)."""
        return self.gemv(Q4_0, packed, N, K, X)

    # -- fp32 activations, SwiGLU ------------------------------------------
    def floats_to_half(self, x: np.ndarray) -> np.ndarray:
        """fp32 activations rounded to binary16 bits (oracle.c's codec)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint16)
        self._L.orc_floats_to_half(self._p(x, ctypes.c_float), x.size, self._p(out, ctypes.c_uint16))
        return out

    def gemv_f32in(self, fmt: int, packed: np.ndarray, N: int, K: int, x32: np.ndarray):
        """(y, s) of the GEMV on fp32 activations rounded to binary16."""
        return self.gemv(fmt, packed, N, K, self.floats_to_half(x32))

    def silu(self, v: float) -> float:
        return float(self._L.orc_silu(float(v)))

    def swiglu(self, packed: np.ndarray, N: int, K: int, x32: np.ndarray):
        """Q4_0 stacked gate + up table (2N x K): (y, g, u, sg, su) with
        y = silu(g) * u, g and u the GEMVs of rows 0..N-1 and N..2N-1 on the
        fp32 activations rounded to binary16, sg and su their sums of |w x|."""
        y2, s2 = self.gemv_f32in(Q4_0, packed, 2 * N, K, x32)
        g = np.ascontiguousarray(y2[:, :N])
        u = np.ascontiguousarray(y2[:, N:])
        y = np.empty_like(g)
        self._L.orc_swiglu(self._p(g, ctypes.c_double), self._p(u, ctypes.c_double), g.size,
                           self._p(y, ctypes.c_double))
        return y, g, u, np.ascontiguousarray(s2[:, :N]), np.ascontiguousarray(s2[:, N:])


    # -- 8-bit activations --------------------------------------------------
    def quantize_act8(self, x: np.ndarray):
        """fp16 activations [M][K] -> (qx int8 [M][K], dx float32 [M][K/32])
        per 32-block (oracle.c: amax / 127, rint(x * 127 / amax), binary32)."""
        x = self._x16(x)
        if x.ndim == 1:
            x = x[None, :]
        M, K = x.shape
        qx = np.empty((M, K), np.int8)
        dx = np.empty((M, K // 32), np.float32)
        self._L.orc_quantize_act8(self._p(x, ctypes.c_uint16), M, K, self._p(qx, ctypes.c_int8),
                                  self._p(dx, ctypes.c_float))
        return qx, dx

    def gemv_q8act_codes(self, packed: np.ndarray, N: int, K: int, qx: np.ndarray, dx: np.ndarray,
                         fmt: int = Q4_0):
        """(y, s) of Q4_0 (or q2w) weights against given 8-bit activations (qx, dx)."""
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        qx = np.ascontiguousarray(qx, dtype=np.int8)
        dx = np.ascontiguousarray(dx, dtype=np.float32)
        M = qx.shape[0]
        assert qx.shape == (M, K) and dx.shape == (M, K // 32)
        y = np.empty((M, N), np.float64)
        s = np.empty((M, N), np.float64)
        assert fmt in (Q4_0, Q2W)
        self._L.orc_gemv_q8act(fmt, self._p(packed, ctypes.c_uint8), N, K, self._p(qx, ctypes.c_int8),
                               self._p(dx, ctypes.c_float), M, self._p(y, ctypes.c_double),
                               self._p(s, ctypes.c_double))
        return y, s

    def gemv_q8act(self, packed: np.ndarray, N: int, K: int, x: np.ndarray, fmt: int = Q4_0):
        """(y, s): the activations quantized to 8-bit blocks, then the GEMV."""
        qx, dx = self.quantize_act8(x)
        return self.gemv_q8act_codes(packed, N, K, qx, dx, fmt)


def within_bound(y, y_ref, s, rel: float = 1e-3, abs_: float = 1e-6):
    """Acceptance bound per element: finite and |y - y_ref| <= rel * s + abs."""
    y = np.asarray(y, dtype=np.float64)
    ok = np.isfinite(y) & (np.abs(y - y_ref) <= rel * s + abs_)
    return ok


def swiglu_within_bound(y, y_ref, g, u, sg, su, rel: float = 1e-3, abs_: float = 1e-6):
    """Acceptance bound of silu(g) u per element, carried from the GEMV bound.

    The kernel's g' and u' satisfy |g' - g| <= eg = rel sg + abs and
    |u' - u| <= eu = rel su + abs.  With L = max |silu'| < 1.1 and
    |silu(g)| <= |g|,
      |silu(g') u' - silu(g) u| <= L eg (|u| + eu) + |g| eu,
    and the fp32 evaluation of silu(g') u' (an exponential, a division and a
    product) adds at most a few units in the last place: 1e-5 |y_ref| + abs.
    """
    y = np.asarray(y, dtype=np.float64)
    eg = rel * sg + abs_
    eu = rel * su + abs_
    bound = 1.1 * eg * (np.abs(u) + eu) + np.abs(g) * eu + 1e-5 * np.abs(y_ref) + abs_
    return np.isfinite(y) & (np.abs(y - y_ref) <= bound)


_default = None


def get() -> Oracle:
    """The shared oracle built from the unmodified source."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
