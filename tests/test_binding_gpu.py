"""The Python binding rejects tensors the kernels would address wrongly (a short,
strided or mistyped output, a vector of the wrong length) before anything is
launched."""
import pytest
import torch

import memory_bound_row_softmax_amd as rr
from _gpu import DEV

pytestmark = pytest.mark.gpu

M, N = 8, 64


def _x(dtype=torch.float32):
    return torch.zeros(M, N, dtype=dtype, device=DEV)


def _f32(n):
    return torch.zeros(n, dtype=torch.float32, device=DEV)


BAD_CALLS = [
    ("softmax y short", lambda: rr.rr_softmax_fwd(_x(), torch.empty(M - 1, N, device=DEV))),
    ("softmax y dtype", lambda: rr.rr_softmax_fwd(_x(), _x(torch.bfloat16))),
    ("softmax y strided", lambda: rr.rr_softmax_fwd(_x(), torch.empty(N, M, device=DEV).t())),
    ("rmsnorm rstd short", lambda: rr.rr_rmsnorm_fwd(_x(), _f32(N), rstd=_f32(M - 1))),
    ("rmsnorm rstd dtype", lambda: rr.rr_rmsnorm_fwd(
        _x(), _f32(N), rstd=torch.zeros(M, dtype=torch.float64, device=DEV))),
    ("rmsnorm w host", lambda: rr.rr_rmsnorm_fwd(_x(), torch.zeros(N))),
    ("xent loss short", lambda: rr.rr_cross_entropy_fwd(
        _x(), torch.zeros(M, dtype=torch.int32, device=DEV), loss=_f32(M - 1))),
    ("xent labels host", lambda: rr.rr_cross_entropy_fwd(_x(), torch.zeros(M, dtype=torch.int32))),
    ("xgrad dlogits shape", lambda: rr.rr_cross_entropy_fwd_bwd(
        _x(), torch.zeros(M, dtype=torch.int32, device=DEV), _f32(M),
        dlogits=torch.empty(M, N - 1, device=DEV))),
    ("xgrad dloss short", lambda: rr.rr_cross_entropy_fwd_bwd(
        _x(), torch.zeros(M, dtype=torch.int32, device=DEV), _f32(M - 1))),
    ("smbwd dx dtype", lambda: rr.rr_softmax_bwd(_x(), _x(), dx=_x(torch.bfloat16))),
    ("smbwd dy shape", lambda: rr.rr_softmax_bwd(_x(), torch.zeros(M, N + 1, device=DEV))),
    ("rmsbwd dw short", lambda: rr.rr_rmsnorm_bwd(_x(), _f32(N), _x(), _f32(M), dw=_f32(N - 1))),
    ("rmsbwd rstd short", lambda: rr.rr_rmsnorm_bwd(_x(), _f32(N), _x(), _f32(M - 1))),
    ("workspace strided", lambda: rr.rr_softmax_fwd(
        _x(), ws=torch.zeros(64, 64, dtype=torch.uint8, device=DEV).t())),
    ("copy strided", lambda: rr.rr_stream_copy(_x(), torch.empty(N, M, device=DEV).t())),
]


@pytest.mark.parametrize("call", BAD_CALLS, ids=lambda c: c[0])
def test_bad_tensors_are_rejected_before_launch(call):
    with pytest.raises(ValueError):
        call[1]()
    torch.cuda.synchronize()


def test_good_outputs_are_accepted():
    x = torch.randn(M, N, device=DEV)
    y = torch.empty_like(x)
    assert rr.rr_softmax_fwd(x, y) is y
    rstd = _f32(M)
    rr.rr_rmsnorm_fwd(x, _f32(N) + 1, rstd=rstd)
    torch.cuda.synchronize()
    assert torch.allclose(y.sum(dim=1), torch.ones(M, device=DEV), atol=1e-5)
    assert bool((rstd > 0).all())
