"""Python binding of libqgemv.so (gfx950): fused dequantize-and-multiply of
block-quantized weights (Q4_0, Q8_0 and plain 2-bit q2w).

This module only marshals arguments: it checks tensor devices, dtypes, shapes
and sizes (the C ABI cannot see buffer sizes), passes raw pointers and the
current HIP stream, and turns a non-zero status into an exception.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
If the library is missing the import of any entry point fails loudly.

Names follow the C ABI in include/qgemv.h.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# QGEMV_LIB points the binding at another build of the library (for example
# a variant compiled for an experiment); default: the in-tree build.
LIB_PATH = os.environ.get("QGEMV_LIB") or os.path.join(_HERE, "libqgemv.so")

QG_STATUS = {0: "ok", 1: "null pointer", 2: "shape out of range", 3: "misaligned pointer",
             4: "non-finite weight or scale overflow", 5: "buffer too small", 6: "kernel launch failed",
             7: "no usable HIP device"}

Q4_0 = 0
Q8_0 = 1
Q2W = 2


class QGError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: status {status} ({QG_STATUS.get(status, 'unknown')})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqgemv.so (after torch, so both use the one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m quantized_weight_gemv_amd.build` "
                          f"(or __graft_entry__.build())")
    try:
        import torch  # noqa: F401  (loads the HIP runtime the library must share)
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "qg_status_str": (ctypes.c_char_p, [c_int]),
        "qpacked_bytes_q4_0": (sz, [i64, i64]),
        "qpacked_bytes_q8_0": (sz, [i64, i64]),
        "qquantize_q4_0": (c_int, [vp, i64, i64, vp, sz]),
        "qquantize_q8_0": (c_int, [vp, i64, i64, vp, sz]),
        "qpacked_bytes_q2w": (sz, [i64, i64]),
        "qquantize_q2w": (c_int, [vp, i64, i64, vp, sz]),
        "qgemv_q2w": (c_int, [vp, vp, vp, c_int, i64, i64, vp]),
        "qgemv_q2w_q8act": (c_int, [vp, vp, vp, c_int, i64, i64, vp]),
        "qgemv_q2w_lut": (c_int, [vp, vp, vp, i64, i64, vp]),
        "qdequant_q2w": (c_int, [vp, i64, i64, c_int, vp, vp]),
        "qgemv_q4_0": (c_int, [vp, vp, vp, c_int, i64, i64, vp]),
        "qgemv_q8_0": (c_int, [vp, vp, vp, c_int, i64, i64, vp]),
        "qgemv_q4_0_f32in": (c_int, [vp, vp, vp, c_int, i64, i64, vp]),
        "qgemv_q4_0_swiglu_f32in": (c_int, [vp, vp, vp, c_int, i64, i64, vp]),
        "qgemv_q4_0_q8act": (c_int, [vp, vp, vp, c_int, i64, i64, vp]),
        "qmoe_gemv_q4_0": (c_int, [vp, i64, vp, vp, vp, c_int, i64, i64, vp]),
        "qgemm_q4_0_prefill": (c_int, [vp, vp, vp, i64, i64, i64, vp]),
        "qdequant_q4_0": (c_int, [vp, i64, i64, c_int, vp, vp]),
        "qdequant_q8_0": (c_int, [vp, i64, i64, c_int, vp, vp]),
        "qg_time_next_launch": (None, [vp, vp]),
        "qg_device_cus": (c_int, [c_int, ctypes.POINTER(c_int)]),
        "qg_set_gemv_shape": (None, [c_int, c_int, c_int, c_int, i64, c_int, c_int, c_int]),
        "qg_read_probe": (c_int, [vp, sz, vp, c_int, c_int, vp]),
        "qg_set_prefill_shape": (None, [c_int, c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def exported_symbols() -> list[str]:
    return ["qg_status_str", "qpacked_bytes_q4_0", "qpacked_bytes_q8_0", "qquantize_q4_0", "qquantize_q8_0",
            "qgemv_q4_0", "qgemv_q8_0", "qgemv_q4_0_f32in", "qgemv_q4_0_swiglu_f32in", "qgemv_q4_0_q8act",
            "qmoe_gemv_q4_0",
            "qgemm_q4_0_prefill", "qdequant_q4_0",
            "qdequant_q8_0", "qpacked_bytes_q2w", "qquantize_q2w", "qgemv_q2w", "qgemv_q2w_q8act", "qgemv_q2w_lut", "qdequant_q2w",
            "qg_time_next_launch", "qg_device_cus", "qg_set_gemv_shape", "qg_read_probe", "qg_set_prefill_shape"]


def _check(fn: str, st: int):
    if st != 0:
        raise QGError(fn, st)


# ------------------------------------------------------------------ host side
def qpacked_bytes_q4_0(N: int, K: int) -> int:
    return int(lib().qpacked_bytes_q4_0(N, K))


def qpacked_bytes_q8_0(N: int, K: int) -> int:
    return int(lib().qpacked_bytes_q8_0(N, K))


def qpacked_bytes_q2w(N: int, K: int) -> int:
    return int(lib().qpacked_bytes_q2w(N, K))


def packed_bytes(fmt: int, N: int, K: int) -> int:
    if fmt == Q2W:
        return qpacked_bytes_q2w(N, K)
    return qpacked_bytes_q4_0(N, K) if fmt == Q4_0 else qpacked_bytes_q8_0(N, K)


def _quantize(fn: str, fmt: int, w: np.ndarray, out: np.ndarray | None) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("weights must be [N][K]")
    N, K = w.shape
    nb = packed_bytes(fmt, N, K)
    if nb == 0:
        raise QGError(fn, 2)
    if out is None:
        out = np.empty(nb, np.uint8)
    if out.dtype != np.uint8 or not out.flags["C_CONTIGUOUS"] or out.size < nb:
        raise ValueError("out must be a contiguous uint8 array of at least the packed size")
    _check(fn, getattr(lib(), fn)(w.ctypes.data, N, K, out.ctypes.data, out.size))
    return out


def qquantize_q4_0(w: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Quantize + pack fp32 [N][K] host weights into the Q4_0 layout (host bytes)."""
    return _quantize("qquantize_q4_0", Q4_0, w, out)


def qquantize_q8_0(w: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Quantize + pack fp32 [N][K] host weights into the Q8_0 layout (host bytes)."""
    return _quantize("qquantize_q8_0", Q8_0, w, out)


def qquantize_q2w(w: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Quantize + pack fp32 [N][K] host weights into the plain 2-bit (q2w) layout."""
    return _quantize("qquantize_q2w", Q2W, w, out)


# ---------------------------------------------------------------- device side
def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dev(t, dtype, name: str, numel: int | None = None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _x16(x):
    torch = _torch()
    if x.dtype == torch.float16:
        return x.view(torch.int16)
    return x


def _gemv(fn: str, fmt: int, Wp, x, N: int, K: int, y=None):
    torch = _torch()
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M][{K}]")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    wp = _dev(Wp, torch.uint8, "Wp", packed_bytes(fmt, N, K))
    xp = _dev(_x16(x), torch.int16, "x", M * K)
    yp = _dev(y, torch.float32, "y", M * N)
    _check(fn, getattr(lib(), fn)(wp, xp, yp, M, N, K, _stream()))
    return y


class PreparedGemv:
    """A qgemv_* call validated once, for launch-bound loops: calling it only
    enqueues the kernel (ctypes call with the stored raw pointers) on the
    stream that was current when it was prepared.  The tensors must stay
    alive and unmoved while the object is used."""

    def __init__(self, fmt: int, Wp, x, y, N: int, K: int):
        torch = _torch()
        if x.dim() != 2 or x.shape[1] != K or y.shape != (x.shape[0], N):
            raise ValueError("x must be [M][K] and y [M][N]")
        self._keep = (Wp, x, y)
        self._name = {Q4_0: "qgemv_q4_0", Q8_0: "qgemv_q8_0", Q2W: "qgemv_q2w"}[fmt]
        self._fn = getattr(lib(), self._name)
        self._args = (_dev(Wp, torch.uint8, "Wp", packed_bytes(fmt, N, K)).value,
                      _dev(_x16(x), torch.int16, "x", x.shape[0] * K).value,
                      _dev(y, torch.float32, "y", x.shape[0] * N).value,
                      int(x.shape[0]), int(N), int(K), _stream().value)

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            raise QGError(self._name, st)


def qgemv_q4_0(Wp, x, N: int, K: int, y=None):
    """y[M][N] (fp32) = dequant(Wp) @ x[M][K]^T; Wp uint8 packed Q4_0, x fp16, 1 <= M <= 8."""
    return _gemv("qgemv_q4_0", Q4_0, Wp, x, N, K, y)


def qgemv_q8_0(Wp, x, N: int, K: int, y=None):
    """y[M][N] (fp32) = dequant(Wp) @ x[M][K]^T; Wp uint8 packed Q8_0, x fp16, 1 <= M <= 8."""
    return _gemv("qgemv_q8_0", Q8_0, Wp, x, N, K, y)


def qgemv_q2w(Wp, x, N: int, K: int, y=None):
    """y[M][N] (fp32) = dequant(Wp) @ x[M][K]^T; Wp uint8 packed q2w, x fp16, 1 <= M <= 8."""
    return _gemv("qgemv_q2w", Q2W, Wp, x, N, K, y)


def qgemv_q2w_q8act(Wp, x, N: int, K: int, y=None):
    """y[M][N] = q2w weights times fp16 x quantized to 8-bit blocks inside the
    launch (int8 dot products); 1 <= M <= 4."""
    return _gemv("qgemv_q2w_q8act", Q2W, Wp, x, N, K, y)


def qgemv_q2w_lut(Wp, x, N: int, K: int, y=None):
    """y[1][N] = q2w weights times one fp16 token through per-pair lookup
    tables in LDS (the times-table design); K <= 4096."""
    torch = _torch()
    if x.dim() != 2 or x.shape != (1, K):
        raise ValueError(f"x must be [1][{K}]")
    if y is None:
        y = torch.empty((1, N), dtype=torch.float32, device=x.device)
    wp = _dev(Wp, torch.uint8, "Wp", packed_bytes(Q2W, N, K))
    xp = _dev(_x16(x), torch.int16, "x", K)
    yp = _dev(y, torch.float32, "y", N)
    _check("qgemv_q2w_lut", lib().qgemv_q2w_lut(wp, xp, yp, N, K, _stream()))
    return y


def qgemv_q4_0_q8act(Wp, x, N: int, K: int, y=None):
    """y[M][N] = Q4_0 weights times fp16 x quantized to 8-bit blocks inside the
    launch (int8 dot products); 1 <= M <= 4."""
    return _gemv("qgemv_q4_0_q8act", Q4_0, Wp, x, N, K, y)


def _f32in(fn: str, Wp, x, N: int, K: int, y, rows: int):
    torch = _torch()
    if x.dim() != 2 or x.shape[1] != K or x.dtype != torch.float32:
        raise ValueError(f"x must be float32 [M][{K}]")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    wp = _dev(Wp, torch.uint8, "Wp", qpacked_bytes_q4_0(rows, K))
    xp = _dev(x, torch.float32, "x", M * K)
    yp = _dev(y, torch.float32, "y", M * N)
    _check(fn, getattr(lib(), fn)(wp, xp, yp, M, N, K, _stream()))
    return y


def qgemv_q4_0_f32in(Wp, x, N: int, K: int, y=None):
    """y[M][N] = dequant(Wp) @ fp16(x)^T with fp32 x rounded inside the kernel; 1 <= M <= 8."""
    return _f32in("qgemv_q4_0_f32in", Wp, x, N, K, y, N)


def qgemv_q4_0_swiglu_f32in(Wp, x, N: int, K: int, y=None):
    """y[M][N] = silu(gate) * up; Wp packs the 2N x K table [gate rows; up rows]."""
    return _f32in("qgemv_q4_0_swiglu_f32in", Wp, x, N, K, y, 2 * N)


def qmoe_gemv_q4_0(pool, P: int, idx, x, N: int, K: int, y=None):
    """y[E][N] = expert idx[e] of the pool times token x[e]; one launch."""
    torch = _torch()
    E = idx.numel()
    if x.dim() != 2 or x.shape != (E, K):
        raise ValueError(f"x must be [E={E}][{K}]")
    if y is None:
        y = torch.empty((E, N), dtype=torch.float32, device=x.device)
    pp = _dev(pool, torch.uint8, "pool", P * qpacked_bytes_q4_0(N, K))
    ip = _dev(idx, torch.int32, "idx", E)
    xp = _dev(_x16(x), torch.int16, "x", E * K)
    yp = _dev(y, torch.float32, "y", E * N)
    _check("qmoe_gemv_q4_0", lib().qmoe_gemv_q4_0(pp, P, ip, xp, yp, E, N, K, _stream()))
    return y


def qgemm_q4_0_prefill(Wp, X, N: int, K: int, Y=None):
    """Y[M][N] (fp32) = X[M][K] @ dequant(Wp)^T on fp16 matrix cores."""
    torch = _torch()
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError(f"X must be [M][{K}]")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    wp = _dev(Wp, torch.uint8, "Wp", qpacked_bytes_q4_0(N, K))
    xp = _dev(_x16(X), torch.int16, "X", M * K)
    yp = _dev(Y, torch.float32, "Y", M * N)
    _check("qgemm_q4_0_prefill", lib().qgemm_q4_0_prefill(wp, xp, yp, M, N, K, _stream()))
    return Y


def _dequant(fn: str, fmt: int, Wp, N: int, K: int, fp16: bool, out=None):
    torch = _torch()
    dt = torch.float16 if fp16 else torch.float32
    if out is None:
        out = torch.empty((N, K), dtype=dt, device=Wp.device)
    wp = _dev(Wp, torch.uint8, "Wp", packed_bytes(fmt, N, K))
    op = _dev(out, dt, "out", N * K)
    _check(fn, getattr(lib(), fn)(wp, N, K, 1 if fp16 else 0, op, _stream()))
    return out


def qdequant_q4_0(Wp, N: int, K: int, fp16: bool = False, out=None):
    return _dequant("qdequant_q4_0", Q4_0, Wp, N, K, fp16, out)


def qdequant_q8_0(Wp, N: int, K: int, fp16: bool = False, out=None):
    return _dequant("qdequant_q8_0", Q8_0, Wp, N, K, fp16, out)


def qdequant_q2w(Wp, N: int, K: int, fp16: bool = False, out=None):
    return _dequant("qdequant_q2w", Q2W, Wp, N, K, fp16, out)


# --------------------------------------------------------------- measurement
def qg_set_gemv_shape(J: int = 0, R: int = 0, ksplit: int = 0, teams_per_wg: int = 0, teams: int = 0,
                      xl: int = -1, engine: int = -1, lanes: int = 0):
    lib().qg_set_gemv_shape(J, R, ksplit, teams_per_wg, teams, xl, engine, lanes)


def qg_read_probe(buf, sink, wgs: int, loads: int = 8, nbytes: int | None = None):
    """Streaming read of the uint8 device tensor `buf` (its first `nbytes`
    bytes, default all) by `wgs` workgroups with `loads` 16-byte loads in
    flight per lane (bandwidth probe)."""
    torch = _torch()
    n = buf.numel() if nbytes is None else int(nbytes)
    bp = _dev(buf, torch.uint8, "buf", n)
    sp = _dev(sink, torch.int32, "sink", wgs)
    _check("qg_read_probe", lib().qg_read_probe(bp, n, sp, wgs, loads, _stream()))


def qg_set_prefill_shape(splits: int = 0, bm: int = 0):
    lib().qg_set_prefill_shape(splits, bm)


def qg_device_cus(device: int = 0) -> int:
    n = ctypes.c_int(0)
    _check("qg_device_cus", lib().qg_device_cus(device, ctypes.byref(n)))
    return n.value


class KernelTimer:
    """HIP events recorded by the kernel launch itself (hipExtLaunchKernel),
    so elapsed() is the kernel's own execution time.  Uses the HIP runtime
    torch already loaded."""

    def __init__(self, count: int):
        self._hip = ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL)
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.start = []
        self.stop = []
        for _ in range(count):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(a)) or self._hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.start.append(a)
            self.stop.append(b)
        self.n = 0

    def arm(self):
        """The next library launch from this thread records into event pair n."""
        i = self.n
        lib().qg_time_next_launch(self.start[i], self.stop[i])
        self.n += 1

    def reset(self):
        self.n = 0

    def elapsed_ms(self) -> list[float]:
        out = []
        for i in range(self.n):
            self._hip.hipEventSynchronize(self.stop[i])
            ms = ctypes.c_float(0)
            rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i])
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            out.append(ms.value)
        return out

    def close(self):
        for e in self.start + self.stop:
            self._hip.hipEventDestroy(e)
        self.start, self.stop = [], []
