"""Python binding of librr (memory-bound row reductions for MI355X / gfx950).

Argument marshalling only: every entry point forwards device pointers, sizes and
the current HIP stream to the C ABI declared in ``include/rr.h``; all arithmetic
runs in the library's HIP kernels.  PyTorch supplies device memory and streams.

The library is loaded from ``librr.so`` next to this file.  If it has not been
built, every call raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
# RR_LIBRARY may name another build of the same sources (tuning runs compare
# builds with different compile-time options); by default the in-tree library.
LIB_PATH = os.environ.get("RR_LIBRARY") or os.path.join(_HERE, "librr.so")

RR_OK = 0
RR_ERR_INVALID_ARGUMENT = 1
RR_ERR_UNSUPPORTED = 2
RR_ERR_WORKSPACE = 3
RR_ERR_HIP = 4
RR_ERR_GRID_TIMEOUT = 5

RR_F32, RR_BF16 = 0, 1
(RR_OP_SOFTMAX, RR_OP_RMSNORM, RR_OP_XENT, RR_OP_XENT_GRAD, RR_OP_SOFTMAX_BWD,
 RR_OP_RMSNORM_BWD) = 0, 1, 2, 3, 4, 5

EXPORTS = ("rr_softmax_fwd", "rr_softmax_fwd_static", "rr_rmsnorm_fwd", "rr_cross_entropy_fwd",
           "rr_cross_entropy_fwd_bwd", "rr_softmax_bwd", "rr_rmsnorm_bwd", "rr_workspace_bytes",
           "rr_workspace_check", "rr_plan_query", "rr_stream_copy", "rr_stream_read_sink_bytes",
           "rr_stream_read", "rr_stream_fill", "rr_set_test_overrides",
           "rr_status_string", "rr_last_hip_error")


class RRError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


class PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("vectorized", ctypes.c_int),
                ("vals_per_lane", ctypes.c_int), ("lanes_per_row", ctypes.c_int),
                ("groups_per_row", ctypes.c_int), ("block_threads", ctypes.c_int),
                ("rows_per_block", ctypes.c_int), ("max_n", ctypes.c_int64),
                ("ws_bytes", ctypes.c_size_t)]


class TestOverrides(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("vals_per_lane", ctypes.c_int),
                ("lanes_per_row", ctypes.c_int), ("groups_per_row", ctypes.c_int),
                ("resident_groups", ctypes.c_int), ("spin_limit", ctypes.c_int)]


_lock = threading.Lock()
_lib = None


def lib():
    """The loaded librr (raises if it is not built).

    PyTorch, when it is installed, is imported first.  Its HIP runtime then serves
    librr too: both carry the soname libamdhip64.so.7, so the dynamic linker resolves
    librr's dependency to the copy already loaded.  Loaded the other way round, librr
    would bring in the system's runtime and torch would still load its own (it names
    the file libamdhip64.so), and torch's memory and streams would reach kernels
    launched through the other runtime."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run "
                                   "`python -m memory_bound_row_softmax_amd.build`")
            try:
                import torch  # noqa: F401  (see above)
            except ImportError:
                pass
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, sz, ci, st = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_int)
            L.rr_softmax_fwd.argtypes = [vp, vp, i64, i64, ci, vp, sz, vp]
            L.rr_softmax_fwd_static.argtypes = [vp, vp, i64, i64, ci, vp]
            L.rr_rmsnorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, ci, ctypes.c_float, vp, sz, vp]
            L.rr_cross_entropy_fwd.argtypes = [vp, vp, vp, vp, i64, i64, ci, vp, sz, vp]
            L.rr_cross_entropy_fwd_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, ci, vp, sz,
                                                   vp]
            L.rr_softmax_bwd.argtypes = [vp, vp, vp, i64, i64, ci, vp, sz, vp]
            L.rr_rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, ci, vp, sz, vp]
            L.rr_workspace_bytes.argtypes = [ci, i64, i64, ci, ci]
            L.rr_workspace_bytes.restype = sz
            L.rr_workspace_check.argtypes = [vp, sz, vp]
            L.rr_plan_query.argtypes = [ci, i64, i64, ci, ci, ctypes.POINTER(PlanInfo)]
            L.rr_stream_copy.argtypes = [vp, vp, sz, vp]
            L.rr_stream_read_sink_bytes.argtypes = [sz]
            L.rr_stream_read_sink_bytes.restype = sz
            L.rr_stream_read.argtypes = [vp, sz, vp, sz, vp]
            L.rr_stream_fill.argtypes = [vp, sz, ctypes.c_uint32, vp]
            L.rr_set_test_overrides.argtypes = [ctypes.POINTER(TestOverrides)]
            L.rr_status_string.argtypes = [ci]
            L.rr_status_string.restype = ctypes.c_char_p
            L.rr_last_hip_error.argtypes = []
            for f in (L.rr_softmax_fwd, L.rr_softmax_fwd_static, L.rr_rmsnorm_fwd, L.rr_cross_entropy_fwd,
                      L.rr_cross_entropy_fwd_bwd, L.rr_softmax_bwd, L.rr_rmsnorm_bwd,
                      L.rr_workspace_check, L.rr_plan_query, L.rr_stream_copy,
                      L.rr_stream_read, L.rr_stream_fill, L.rr_set_test_overrides,
                      L.rr_last_hip_error):
                f.restype = st
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().rr_status_string(status).decode()


def _check(status: int, what: str):
    if status != RR_OK:
        raise RRError(status, what)


# --------------------------------------------------------------- raw pointers
# The same entry points with plain integers (device addresses, stream handle),
# for callers that manage memory themselves (the bench).

def softmax_fwd_raw(x, y, M, N, dt, ws=0, ws_bytes=0, stream=0) -> int:
    return lib().rr_softmax_fwd(x, y, M, N, dt, ws or None, ws_bytes, stream or None)


def softmax_fwd_static_raw(x, y, M, N, dt, stream=0) -> int:
    """rr_softmax_fwd_static: the split-row workspace is the library's own."""
    return lib().rr_softmax_fwd_static(x, y, M, N, dt, stream or None)


def rmsnorm_fwd_raw(x, w, y, rstd, M, N, dt, eps, ws=0, ws_bytes=0, stream=0) -> int:
    return lib().rr_rmsnorm_fwd(x, w, y, rstd or None, M, N, dt, eps, ws or None, ws_bytes,
                                stream or None)


def cross_entropy_fwd_raw(x, labels, loss, lse, M, N, dt, ws=0, ws_bytes=0, stream=0) -> int:
    return lib().rr_cross_entropy_fwd(x, labels, loss, lse or None, M, N, dt, ws or None,
                                      ws_bytes, stream or None)


def cross_entropy_fwd_bwd_raw(x, labels, dloss, loss, lse, dx, M, N, dt, ws=0, ws_bytes=0,
                              stream=0) -> int:
    return lib().rr_cross_entropy_fwd_bwd(x, labels, dloss, loss, lse or None, dx, M, N, dt,
                                          ws or None, ws_bytes, stream or None)


def softmax_bwd_raw(y, dy, dx, M, N, dt, ws=0, ws_bytes=0, stream=0) -> int:
    return lib().rr_softmax_bwd(y, dy, dx, M, N, dt, ws or None, ws_bytes, stream or None)


def rmsnorm_bwd_raw(x, w, dy, rstd, dx, dw, M, N, dt, ws=0, ws_bytes=0, stream=0) -> int:
    return lib().rr_rmsnorm_bwd(x, w, dy, rstd, dx, dw, M, N, dt, ws or None, ws_bytes,
                                stream or None)


def stream_copy_raw(src, dst, nbytes, stream=0) -> int:
    return lib().rr_stream_copy(src, dst, nbytes, stream or None)


def stream_read_sink_bytes(nbytes) -> int:
    return int(lib().rr_stream_read_sink_bytes(nbytes))


def stream_read_raw(src, nbytes, sink, sink_bytes, stream=0) -> int:
    return lib().rr_stream_read(src, nbytes, sink, sink_bytes, stream or None)


def stream_fill_raw(dst, nbytes, value, stream=0) -> int:
    return lib().rr_stream_fill(dst, nbytes, value & 0xFFFFFFFF, stream or None)


# --------------------------------------------------------------- torch tensors

def _torch():
    import torch

    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RR_F32
    if t.dtype == torch.bfloat16:
        return RR_BF16
    raise TypeError(f"librr takes float32 or bfloat16 tensors, got {t.dtype}")


def _handle(stream) -> int:
    """A raw stream handle from a torch stream or an integer handle."""
    return int(getattr(stream, "cuda_stream", stream))


def _stream(t, stream):
    if stream is not None:
        return _handle(stream)
    return _torch().cuda.current_stream(t.device).cuda_stream


class _on_stream:
    """Makes the launch stream current while a call allocates its outputs and
    workspace, so that they are allocated (and the workspace zero-filled) in that
    stream's order: the zero fill then precedes the kernel, and the caching allocator
    does not hand the memory to other work before the kernel is done with it.
    Yields the raw handle of the launch stream."""

    def __init__(self, device, stream):
        self.device, self.stream, self.ctx = device, stream, None

    def __enter__(self) -> int:
        torch = _torch()
        cur = torch.cuda.current_stream(self.device)
        if self.stream is None or _handle(self.stream) == cur.cuda_stream:
            return cur.cuda_stream
        ext = (self.stream if isinstance(self.stream, torch.cuda.Stream)
               else torch.cuda.ExternalStream(_handle(self.stream), device=self.device))
        self.ctx = torch.cuda.stream(ext)
        self.ctx.__enter__()
        return ext.cuda_stream

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.__exit__(*exc)
        return False


def _matrix(x):
    if x.dim() != 2 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("expected a contiguous 2-D CUDA tensor [M, N]")
    return x.shape[0], x.shape[1]


def _like(t, ref, name):
    """An output (or second input) the kernels address as ref's shape and dtype."""
    if (t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous()
            or t.device != ref.device):
        raise ValueError(f"{name} must be a contiguous tensor of shape {tuple(ref.shape)}, "
                         f"dtype {ref.dtype} on {ref.device}")
    return t


def _f32_vector(t, n, device, name):
    """A contiguous fp32 vector of n elements on `device` (rstd, loss, lse, dloss, dw)."""
    import torch

    if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 [{n}] tensor on {device}")
    return t


def workspace_bytes(op: int, M: int, N: int, dt: int) -> int:
    return int(lib().rr_workspace_bytes(op, M, N, dt, -1))


def workspace(op: int, M: int, N: int, dt: int, device):
    """A zero-filled workspace for this call shape, or None when none is needed."""
    n = workspace_bytes(op, M, N, dt)
    if n == 0:
        return None
    return _torch().zeros(n, dtype=_torch().uint8, device=device)


def _ws_args(ws):
    if ws is None:
        return 0, 0
    if not ws.is_contiguous() or not ws.is_cuda:
        raise ValueError("the workspace must be a contiguous CUDA tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def rr_softmax_fwd(x, y=None, ws=None, stream=None):
    """Row softmax of x [M, N] into y (new tensor if None; y may be x)."""
    M, N = _matrix(x)
    dt = dtype_code(x)
    with _on_stream(x.device, stream) as sp:
        y = _torch().empty_like(x) if y is None else _like(y, x, "y")
        if ws is None:
            ws = workspace(RR_OP_SOFTMAX, M, N, dt, x.device)
        wp, wb = _ws_args(ws)
        _check(softmax_fwd_raw(x.data_ptr(), y.data_ptr(), M, N, dt, wp, wb, sp),
               "rr_softmax_fwd")
    return y


def rr_rmsnorm_fwd(x, w, eps=1e-6, y=None, rstd=None, ws=None, stream=None):
    """RMSNorm of x [M, N] with weight w [N]; returns y (and fills rstd [M] if given)."""
    M, N = _matrix(x)
    if w.dtype != x.dtype or w.numel() != N or not w.is_contiguous() or w.device != x.device:
        raise ValueError("weight must be a contiguous [N] tensor of the input's dtype")
    if rstd is not None:
        _f32_vector(rstd, M, x.device, "rstd")
    dt = dtype_code(x)
    with _on_stream(x.device, stream) as sp:
        y = _torch().empty_like(x) if y is None else _like(y, x, "y")
        if ws is None:
            ws = workspace(RR_OP_RMSNORM, M, N, dt, x.device)
        wp, wb = _ws_args(ws)
        _check(rmsnorm_fwd_raw(x.data_ptr(), w.data_ptr(), y.data_ptr(),
                               rstd.data_ptr() if rstd is not None else 0, M, N, dt, float(eps),
                               wp, wb, sp), "rr_rmsnorm_fwd")
    return y


def rr_cross_entropy_fwd(logits, labels, loss=None, lse=None, ws=None, stream=None):
    """Per-row cross-entropy of logits [M, N] with int32 labels [M]; returns (loss, lse)."""
    torch = _torch()
    M, N = _matrix(logits)
    if labels.dtype != torch.int32 or labels.numel() != M or not labels.is_contiguous():
        raise ValueError("labels must be a contiguous int32 [M] tensor")
    if labels.device != logits.device:
        raise ValueError("labels must be on the logits' device")
    dt = dtype_code(logits)
    with _on_stream(logits.device, stream) as sp:
        loss = (torch.empty(M, dtype=torch.float32, device=logits.device) if loss is None
                else _f32_vector(loss, M, logits.device, "loss"))
        lse = (torch.empty(M, dtype=torch.float32, device=logits.device) if lse is None
               else _f32_vector(lse, M, logits.device, "lse"))
        wp, wb = _ws_args(ws)
        _check(cross_entropy_fwd_raw(logits.data_ptr(), labels.data_ptr(), loss.data_ptr(),
                                     lse.data_ptr(), M, N, dt, wp, wb, sp),
               "rr_cross_entropy_fwd")
    return loss, lse


def rr_cross_entropy_fwd_bwd(logits, labels, dloss, dlogits=None, loss=None, lse=None, ws=None,
                             stream=None):
    """Per-row cross-entropy of logits [M, N] (int32 labels [M]) and its gradient
    dlogits = (softmax - onehot) * dloss[:, None] (fp32 dloss [M]); dlogits may be
    logits itself.  Returns (loss, lse, dlogits)."""
    torch = _torch()
    M, N = _matrix(logits)
    if labels.dtype != torch.int32 or labels.numel() != M or not labels.is_contiguous():
        raise ValueError("labels must be a contiguous int32 [M] tensor")
    if labels.device != logits.device:
        raise ValueError("labels must be on the logits' device")
    _f32_vector(dloss, M, logits.device, "dloss")
    dt = dtype_code(logits)
    with _on_stream(logits.device, stream) as sp:
        dlogits = (torch.empty_like(logits) if dlogits is None
                   else _like(dlogits, logits, "dlogits"))
        loss = (torch.empty(M, dtype=torch.float32, device=logits.device) if loss is None
                else _f32_vector(loss, M, logits.device, "loss"))
        lse = (torch.empty(M, dtype=torch.float32, device=logits.device) if lse is None
               else _f32_vector(lse, M, logits.device, "lse"))
        if ws is None:
            ws = workspace(RR_OP_XENT_GRAD, M, N, dt, logits.device)
        wp, wb = _ws_args(ws)
        _check(cross_entropy_fwd_bwd_raw(logits.data_ptr(), labels.data_ptr(), dloss.data_ptr(),
                                         loss.data_ptr(), lse.data_ptr(), dlogits.data_ptr(), M,
                                         N, dt, wp, wb, sp), "rr_cross_entropy_fwd_bwd")
    return loss, lse, dlogits


def rr_softmax_bwd(y, dy, dx=None, ws=None, stream=None):
    """Softmax backward from the forward output y [M, N] and the gradient dy [M, N]:
    dx = y * (dy - rowsum(y * dy)); dx may be y or dy itself."""
    M, N = _matrix(y)
    _like(dy, y, "dy")
    dt = dtype_code(y)
    with _on_stream(y.device, stream) as sp:
        dx = _torch().empty_like(y) if dx is None else _like(dx, y, "dx")
        if ws is None:
            ws = workspace(RR_OP_SOFTMAX_BWD, M, N, dt, y.device)
        wp, wb = _ws_args(ws)
        _check(softmax_bwd_raw(y.data_ptr(), dy.data_ptr(), dx.data_ptr(), M, N, dt, wp, wb, sp),
               "rr_softmax_bwd")
    return dx


def rr_rmsnorm_bwd(x, w, dy, rstd, dx=None, dw=None, ws=None, stream=None):
    """RMSNorm backward from x [M, N], w [N], dy [M, N] and the forward's fp32 rstd [M];
    returns (dx [M, N] of x's dtype, dw [N] fp32).  dx may be x or dy itself."""
    torch = _torch()
    M, N = x.shape if x.dim() == 2 else (None, None)
    if M is None or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("expected a contiguous 2-D CUDA tensor [M, N]")
    _like(dy, x, "dy")
    if w.dtype != x.dtype or w.numel() != N or not w.is_contiguous() or w.device != x.device:
        raise ValueError("weight must be a contiguous [N] tensor of the input's dtype")
    _f32_vector(rstd, M, x.device, "rstd")
    dt = dtype_code(x)
    with _on_stream(x.device, stream) as sp:
        dx = torch.empty_like(x) if dx is None else _like(dx, x, "dx")
        dw = (torch.empty(N, dtype=torch.float32, device=x.device) if dw is None
              else _f32_vector(dw, N, x.device, "dw"))
        if ws is None:
            ws = workspace(RR_OP_RMSNORM_BWD, M, N, dt, x.device)
        wp, wb = _ws_args(ws)
        _check(rmsnorm_bwd_raw(x.data_ptr(), w.data_ptr(), dy.data_ptr(), rstd.data_ptr(),
                               dx.data_ptr(), dw.data_ptr(), M, N, dt, wp, wb, sp),
               "rr_rmsnorm_bwd")
    return dx, dw


def rr_workspace_check(ws, stream=None) -> int:
    """Synchronises the stream and returns (and clears) the workspace's status:
    RR_OK, or RR_ERR_GRID_TIMEOUT if a split row of a launch that used `ws` gave up
    waiting for its peer workgroups (that row's outputs are then NaN).  The ops above
    do not call it themselves (it synchronises); a caller that passes its own `ws`
    checks it when it synchronises anyway."""
    wp, wb = _ws_args(ws)
    return lib().rr_workspace_check(wp, wb, _stream(ws, stream))


_KINDS = {None: 0, "block": 1, "stream": 2, "long": 3}


def set_test_overrides(kind=None, P=None, R=None, G=None, groups=None, spin=None):
    """Test-only: forces the plan (kernel kind, P, R, G), the row groups of a persistent
    grid and the bound of each split-row wait (spin = -1: every wait gives up) for every
    later call in the process; with no arguments, restores the defaults.  See
    rr_set_test_overrides in include/rr.h."""
    o = TestOverrides(_KINDS[kind], P or 0, R or 0, G or 0, groups or 0, spin or 0)
    _check(lib().rr_set_test_overrides(ctypes.byref(o)), "rr_set_test_overrides")


def rr_stream_copy(src, dst, stream=None):
    """Copies src into dst (the same-run copy ceiling of the bench)."""
    if not (src.is_contiguous() and dst.is_contiguous() and src.is_cuda and dst.is_cuda
            and src.device == dst.device):
        raise ValueError("src and dst must be contiguous CUDA tensors on one device")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("destination too small")
    _check(stream_copy_raw(src.data_ptr(), dst.data_ptr(), nbytes, _stream(src, stream)),
           "rr_stream_copy")
    return dst


def rr_plan_query(op: int, M: int, N: int, dt: int, vectorized: bool = True) -> dict:
    info = PlanInfo()
    _check(lib().rr_plan_query(op, M, N, dt, 1 if vectorized else 0, ctypes.byref(info)),
           "rr_plan_query")
    return {k: getattr(info, k) for k, _ in PlanInfo._fields_}
