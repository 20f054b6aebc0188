"""Python access to the plain CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
CPU-baseline leg of the benchmark are the only callers.  The GPU library and
its Python binding never import this package.

The oracle is built with gcc (no fast-math, no FP contraction, OpenMP over
output rows) into ``liboracle.so`` beside this file.  ``Oracle(path)`` loads
any build of it, which lets a test load a deliberately broken copy.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


def build(out: str = LIB, src: str = SRC, extra=()) -> str:
    """Compile oracle.c (or another source) into a shared library."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


# weight formats (the oracle's own numbering)
FMT_IQ4_XS, FMT_IQ4_NL, FMT_Q4_0 = 0, 1, 2

_p = ctypes.c_void_p
_i64 = ctypes.c_int64


class Oracle:
    """ctypes wrapper around one build of the oracle library."""

    def __init__(self, path: str = LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_float_to_half.argtypes = [ctypes.c_float]
        lib.oracle_float_to_half.restype = ctypes.c_uint16
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_kvalue.argtypes = [ctypes.c_int]
        lib.oracle_kvalue.restype = ctypes.c_int
        for name in ("oracle_dequantize", "oracle_dequantize_bf16"):
            getattr(lib, name).argtypes = [_p, _i64, _i64, _p]
            getattr(lib, name).restype = None
        lib.oracle_quantize_q8_1.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_quantize_q8_1.restype = None
        for name in ("oracle_gemm_q8_1", "oracle_gemm_bf16", "oracle_gemm_bf16x3"):
            getattr(lib, name).argtypes = [_p, _p, _i64, _i64, _i64, _p]
            getattr(lib, name).restype = None
        for name in ("oracle_float_to_half_array", "oracle_half_to_double_array",
                     "oracle_double_to_bf16_array"):
            getattr(lib, name).argtypes = [_p, _i64, _p]
            getattr(lib, name).restype = None
        lib.oracle_row_bytes.argtypes = [ctypes.c_int, _i64]
        lib.oracle_row_bytes.restype = _i64
        lib.oracle_dequantize_fmt.argtypes = [ctypes.c_int, _p, _i64, _i64, _p]
        lib.oracle_dequantize_fmt.restype = None
        lib.oracle_gemm_fmt_q8_1.argtypes = [ctypes.c_int, _p, _p, _i64, _i64, _i64, _p]
        lib.oracle_gemm_fmt_q8_1.restype = None
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        lib.oracle_get_threads.argtypes = []
        lib.oracle_get_threads.restype = ctypes.c_int
        self.lib = lib

    # -- scalar helpers -------------------------------------------------
    def half_to_double(self, h: int) -> float:
        return self.lib.oracle_half_to_double(int(h))

    def float_to_half(self, x: float) -> int:
        return self.lib.oracle_float_to_half(float(np.float32(x)))

    def double_to_bf16(self, x: float) -> int:
        return self.lib.oracle_double_to_bf16(float(x))

    def float_to_half_array(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_float_to_half_array(x.ctypes.data, x.size, out.ctypes.data)
        return out

    def half_to_double_array(self, h: np.ndarray) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16)
        out = np.empty(h.shape, dtype=np.float64)
        self.lib.oracle_half_to_double_array(h.ctypes.data, h.size, out.ctypes.data)
        return out

    def double_to_bf16_array(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_double_to_bf16_array(x.ctypes.data, x.size, out.ctypes.data)
        return out

    def kvalues(self) -> np.ndarray:
        return np.array([self.lib.oracle_kvalue(i) for i in range(16)], dtype=np.int64)

    def set_threads(self, t: int) -> None:
        self.lib.oracle_set_threads(int(t))

    def threads(self) -> int:
        return self.lib.oracle_get_threads()

    # -- array functions ------------------------------------------------
    @staticmethod
    def _wcheck(W: np.ndarray, K: int) -> tuple:
        if K % 256:
            raise ValueError("K must be a multiple of 256")
        W = np.ascontiguousarray(W, dtype=np.uint8)
        if W.ndim != 2 or W.shape[1] != (K // 256) * 136:
            raise ValueError("W must be uint8 [N, K/256*136]")
        return W, W.shape[0]

    @staticmethod
    def _xqcheck(Xq: np.ndarray, K: int) -> tuple:
        Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
        if Xq.ndim != 2 or Xq.shape[1] != (K // 32) * 36:
            raise ValueError("Xq must be uint8 [M, K/32*36]")
        return Xq, Xq.shape[0]

    def dequantize(self, W: np.ndarray, K: int) -> np.ndarray:
        W, N = self._wcheck(W, K)
        out = np.empty((N, K), dtype=np.float64)
        self.lib.oracle_dequantize(W.ctypes.data, N, K, out.ctypes.data)
        return out

    def dequantize_bf16(self, W: np.ndarray, K: int) -> np.ndarray:
        W, N = self._wcheck(W, K)
        out = np.empty((N, K), dtype=np.uint16)
        self.lib.oracle_dequantize_bf16(W.ctypes.data, N, K, out.ctypes.data)
        return out

    def quantize_q8_1(self, X: np.ndarray) -> np.ndarray:
        X = np.ascontiguousarray(X, dtype=np.float32)
        M, K = X.shape
        if K % 32:
            raise ValueError("K must be a multiple of 32")
        out = np.empty((M, (K // 32) * 36), dtype=np.uint8)
        self.lib.oracle_quantize_q8_1(X.ctypes.data, M, K, out.ctypes.data)
        return out

    def gemm_q8_1(self, W: np.ndarray, Xq: np.ndarray, K: int) -> np.ndarray:
        W, N = self._wcheck(W, K)
        Xq, M = self._xqcheck(Xq, K)
        Y = np.empty((M, N), dtype=np.float64)
        self.lib.oracle_gemm_q8_1(W.ctypes.data, Xq.ctypes.data, M, N, K, Y.ctypes.data)
        return Y

    def gemm_bf16(self, W: np.ndarray, Xq: np.ndarray, K: int) -> np.ndarray:
        W, N = self._wcheck(W, K)
        Xq, M = self._xqcheck(Xq, K)
        Y = np.empty((M, N), dtype=np.float64)
        self.lib.oracle_gemm_bf16(W.ctypes.data, Xq.ctypes.data, M, N, K, Y.ctypes.data)
        return Y

    def gemm_bf16x3(self, W: np.ndarray, Xq: np.ndarray, K: int) -> np.ndarray:
        """Compensated bf16 formulation: W~ and X~ each split into bf16 hi
        and lo parts, Wh*Xh + Wh*Xl + Wl*Xh summed exactly."""
        W, N = self._wcheck(W, K)
        Xq, M = self._xqcheck(Xq, K)
        Y = np.empty((M, N), dtype=np.float64)
        self.lib.oracle_gemm_bf16x3(W.ctypes.data, Xq.ctypes.data, M, N, K, Y.ctypes.data)
        return Y

    def gemm(self, W: np.ndarray, X: np.ndarray) -> np.ndarray:
        """Quantize fp32 X to Q8_1, then the integer-dot GEMM."""
        K = X.shape[1]
        return self.gemm_q8_1(W, self.quantize_q8_1(X), K)

    # -- other weight formats (FMT_IQ4_XS, FMT_IQ4_NL, FMT_Q4_0) --------
    def row_bytes(self, fmt: int, K: int) -> int:
        return self.lib.oracle_row_bytes(int(fmt), int(K))

    def _wcheck_fmt(self, fmt: int, W: np.ndarray, K: int) -> tuple:
        rb = self.row_bytes(fmt, K)
        if rb <= 0 or K % (256 if fmt == FMT_IQ4_XS else 32):
            raise ValueError("unknown format or K not a whole number of blocks")
        W = np.ascontiguousarray(W, dtype=np.uint8)
        if W.ndim != 2 or W.shape[1] != rb:
            raise ValueError(f"W must be uint8 [N, {rb}]")
        return W, W.shape[0]

    def dequantize_fmt(self, fmt: int, W: np.ndarray, K: int) -> np.ndarray:
        W, N = self._wcheck_fmt(fmt, W, K)
        out = np.empty((N, K), dtype=np.float64)
        self.lib.oracle_dequantize_fmt(int(fmt), W.ctypes.data, N, K, out.ctypes.data)
        return out

    def gemm_fmt_q8_1(self, fmt: int, W: np.ndarray, Xq: np.ndarray, K: int) -> np.ndarray:
        W, N = self._wcheck_fmt(fmt, W, K)
        Xq, M = self._xqcheck(Xq, K)
        Y = np.empty((M, N), dtype=np.float64)
        self.lib.oracle_gemm_fmt_q8_1(int(fmt), W.ctypes.data, Xq.ctypes.data, M, N, K, Y.ctypes.data)
        return Y

    def gemm_fmt(self, fmt: int, W: np.ndarray, X: np.ndarray) -> np.ndarray:
        K = X.shape[1]
        return self.gemm_fmt_q8_1(fmt, W, self.quantize_q8_1(X), K)


_default = None


def get() -> Oracle:
    """The oracle built from oracle.c beside this file (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default
