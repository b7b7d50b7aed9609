"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the bench.

This package only draws numbers (see ``synth.c`` for the generator's
definition); it holds none of the arithmetic of the three row reductions.
Arrays come back as numpy: float32 for fp32 data, uint16 bit patterns for
bf16 data, int32 for labels.  Any subset of rows can be regenerated on its
own (``rows=[...]``) and equals the same rows of a full draw.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

SEED = 0x5EED
STREAM_X, STREAM_W, STREAM_LABELS, STREAM_SPIKES = 0, 1, 2, 3
# upstream gradients of the backward passes: dy (per element), dloss (per row)
STREAM_DY, STREAM_DLOSS = 4, 5
DTYPES = {"f32": 0, "bf16": 1}

_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile ``libsynth.so`` next to its source with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"],
                   check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
            i64, u64, dbl, vp, ci = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_double,
                                     ctypes.c_void_p, ctypes.c_int)
            for name in ("synth_normal", "synth_uniform", "synth_spikes"):
                f = getattr(lib, name)
                f.argtypes = [u64, u64, vp, i64, i64, i64, dbl, dbl, ci, vp, ci]
                f.restype = None
            lib.synth_labels.argtypes = [u64, u64, vp, i64, i64, i64, vp]
            lib.synth_labels.restype = None
            lib.synth_f32_to_bf16.argtypes = [vp, vp, i64]
            lib.synth_f32_to_bf16.restype = None
            _lib = lib
    return _lib


def _np_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _rows_arg(rows):
    if rows is None:
        return None, None
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, r.ctypes.data


def _fill(fn, M, N, a, b, dtype, seed, stream, row0, rows, nthreads, out):
    r, rp = _rows_arg(rows)
    nrows = M if r is None else len(r)
    if out is None:
        out = np.empty((nrows, N), dtype=_np_dtype(dtype))
    assert out.flags.c_contiguous and out.shape == (nrows, N) and out.dtype == _np_dtype(dtype)
    fn(seed, stream, rp, row0, nrows, N, a, b, DTYPES[dtype], out.ctypes.data, nthreads)
    return out


def normal(M, N, *, sigma=1.0, mean=0.0, dtype="f32", seed=SEED, stream=STREAM_X, row0=0,
           rows=None, nthreads=0, out=None):
    """mean + sigma * N(0,1), shape (M or len(rows), N)."""
    return _fill(_load().synth_normal, M, N, sigma, mean, dtype, seed, stream, row0, rows,
                 nthreads, out)


def uniform(M, N, *, lo=0.0, hi=1.0, dtype="f32", seed=SEED, stream=STREAM_W, row0=0,
            rows=None, nthreads=0, out=None):
    """U(lo, hi), shape (M or len(rows), N)."""
    return _fill(_load().synth_uniform, M, N, lo, hi, dtype, seed, stream, row0, rows,
                 nthreads, out)


def spikes_(x, *, p=0.01, value=20.0, dtype="f32", seed=SEED, stream=STREAM_SPIKES, row0=0,
            rows=None, nthreads=0):
    """In place: each element independently becomes ``value`` with probability p."""
    M, N = x.shape
    _fill(_load().synth_spikes, M, N, p, value, dtype, seed, stream, row0, rows, nthreads, x)
    return x


def labels(M, N, *, seed=SEED, stream=STREAM_LABELS, row0=0, rows=None):
    """One int32 label per row, uniform in [0, N)."""
    r, rp = _rows_arg(rows)
    nrows = M if r is None else len(r)
    out = np.empty(nrows, dtype=np.int32)
    _load().synth_labels(seed, stream, rp, row0, nrows, N, out.ctypes.data)
    return out


def f32_to_bf16(a) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out


from . import workloads  # noqa: E402,F401  (input recipes of the benchmarked configurations)
