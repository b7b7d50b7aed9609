"""ctypes binding of the double-precision CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()``
and by the bench's CPU-baseline leg, never by the GPU library or its binding.

Inputs are numpy arrays: float32 for fp32 data, uint16 bit patterns for bf16
data, int32 labels.  Outputs are float64 arrays holding the unrounded results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CODES = {"f32": 0, "bf16": 1}
_lock = threading.Lock()
_lib = None


def compile_library(src: str, out: str) -> str:
    """gcc -O2 a copy of the oracle source into a shared library at ``out``."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile ``liboracle.so`` next to its source (always recompiles)."""
    return compile_library(_SRC, _LIB)


def bind(path: str):
    """Load an oracle library (the real one, or a test's planted-mistake copy)."""
    lib = ctypes.CDLL(path)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_softmax.argtypes = [vp, ci, i64, i64, vp]
    lib.oracle_rmsnorm.argtypes = [vp, vp, ci, i64, i64, ctypes.c_float, vp, vp]
    lib.oracle_cross_entropy.argtypes = [vp, vp, ci, i64, i64, vp, vp]
    lib.oracle_cross_entropy_grad.argtypes = [vp, vp, vp, ci, i64, i64, vp, vp, vp]
    lib.oracle_softmax_backward.argtypes = [vp, vp, ci, i64, i64, vp]
    lib.oracle_rmsnorm_backward.argtypes = [vp, vp, vp, vp, ci, i64, i64, vp, vp]
    for f in (lib.oracle_softmax, lib.oracle_rmsnorm, lib.oracle_cross_entropy,
              lib.oracle_cross_entropy_grad, lib.oracle_softmax_backward,
              lib.oracle_rmsnorm_backward):
        f.restype = ci
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            _lib = bind(_LIB)
    return _lib


def _dtype_of(x: np.ndarray) -> str:
    if x.dtype == np.float32:
        return "f32"
    if x.dtype == np.uint16:
        return "bf16"
    raise TypeError(f"oracle inputs are float32 or uint16 (bf16 bits), got {x.dtype}")


class Oracle:
    """The reference functions, bound to one compiled oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else _load()

    def softmax(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x)
        M, N = x.shape
        y = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_softmax(x.ctypes.data, _CODES[_dtype_of(x)], M, N, y.ctypes.data)
        if rc:
            raise ValueError("oracle_softmax rejected its arguments")
        return y

    def rmsnorm(self, x: np.ndarray, w: np.ndarray, eps: float, want_rstd: bool = False):
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        M, N = x.shape
        if w.dtype != x.dtype or w.shape != (N,):
            raise ValueError("weight must have shape (N,) and the input's dtype")
        y = np.empty((M, N), dtype=np.float64)
        rstd = np.empty(M, dtype=np.float64)
        rc = self.lib.oracle_rmsnorm(x.ctypes.data, w.ctypes.data, _CODES[_dtype_of(x)], M, N,
                                     float(eps), y.ctypes.data, rstd.ctypes.data)
        if rc:
            raise ValueError("oracle_rmsnorm rejected its arguments")
        return (y, rstd) if want_rstd else y

    def cross_entropy(self, x: np.ndarray, labels: np.ndarray):
        """Returns (loss[M], lse[M]) in float64."""
        x = np.ascontiguousarray(x)
        labels = np.ascontiguousarray(labels, dtype=np.int32)
        M, N = x.shape
        if labels.shape != (M,):
            raise ValueError("labels must have shape (M,)")
        loss = np.empty(M, dtype=np.float64)
        lse = np.empty(M, dtype=np.float64)
        rc = self.lib.oracle_cross_entropy(x.ctypes.data, labels.ctypes.data,
                                           _CODES[_dtype_of(x)], M, N, loss.ctypes.data,
                                           lse.ctypes.data)
        if rc:
            raise ValueError("oracle_cross_entropy rejected its arguments")
        return loss, lse

    def cross_entropy_grad(self, x: np.ndarray, labels: np.ndarray, dloss: np.ndarray):
        """Returns (loss[M], lse[M], dx[M, N]) in float64; dloss is float32[M]."""
        x = np.ascontiguousarray(x)
        labels = np.ascontiguousarray(labels, dtype=np.int32)
        dloss = np.ascontiguousarray(dloss, dtype=np.float32)
        M, N = x.shape
        if labels.shape != (M,) or dloss.shape != (M,):
            raise ValueError("labels and dloss must have shape (M,)")
        loss = np.empty(M, dtype=np.float64)
        lse = np.empty(M, dtype=np.float64)
        dx = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_cross_entropy_grad(x.ctypes.data, labels.ctypes.data,
                                                dloss.ctypes.data, _CODES[_dtype_of(x)], M, N,
                                                loss.ctypes.data, lse.ctypes.data, dx.ctypes.data)
        if rc:
            raise ValueError("oracle_cross_entropy_grad rejected its arguments")
        return loss, lse, dx

    def softmax_backward(self, y: np.ndarray, dy: np.ndarray) -> np.ndarray:
        """dx[M, N] in float64 from the forward output y and the gradient dy."""
        y = np.ascontiguousarray(y)
        dy = np.ascontiguousarray(dy)
        M, N = y.shape
        if dy.dtype != y.dtype or dy.shape != (M, N):
            raise ValueError("dy must have the shape and dtype of y")
        dx = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_softmax_backward(y.ctypes.data, dy.ctypes.data, _CODES[_dtype_of(y)],
                                              M, N, dx.ctypes.data)
        if rc:
            raise ValueError("oracle_softmax_backward rejected its arguments")
        return dx

    def rmsnorm_backward(self, x: np.ndarray, w: np.ndarray, dy: np.ndarray, rstd: np.ndarray):
        """(dx[M, N], dw[N]) in float64; rstd is the forward's float32[M]."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        dy = np.ascontiguousarray(dy)
        rstd = np.ascontiguousarray(rstd, dtype=np.float32)
        M, N = x.shape
        if w.dtype != x.dtype or w.shape != (N,) or dy.dtype != x.dtype or dy.shape != (M, N):
            raise ValueError("w must be (N,) and dy (M, N), both of the input's dtype")
        if rstd.shape != (M,):
            raise ValueError("rstd must have shape (M,)")
        dx = np.empty((M, N), dtype=np.float64)
        dw = np.empty(N, dtype=np.float64)
        rc = self.lib.oracle_rmsnorm_backward(x.ctypes.data, w.ctypes.data, dy.ctypes.data,
                                              rstd.ctypes.data, _CODES[_dtype_of(x)], M, N,
                                              dx.ctypes.data, dw.ctypes.data)
        if rc:
            raise ValueError("oracle_rmsnorm_backward rejected its arguments")
        return dx, dw


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def softmax(x):
    return default().softmax(x)


def rmsnorm(x, w, eps, want_rstd=False):
    return default().rmsnorm(x, w, eps, want_rstd)


def cross_entropy(x, labels):
    return default().cross_entropy(x, labels)


def cross_entropy_grad(x, labels, dloss):
    return default().cross_entropy_grad(x, labels, dloss)


def softmax_backward(y, dy):
    return default().softmax_backward(y, dy)


def rmsnorm_backward(x, w, dy, rstd):
    return default().rmsnorm_backward(x, w, dy, rstd)
