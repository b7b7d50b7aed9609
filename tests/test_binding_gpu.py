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


def test_calls_on_a_stream_that_is_not_current():
    """Outputs and the workspace the binding allocates are made in the launch
    stream's order (so the zero fill precedes the kernel, and the memory is not handed
    to other work while the kernel runs): split rows on a side stream, while the
    current stream is busy, give the right rows and a clean status."""
    import numpy as np

    import oracle
    import synth
    from _gpu import from_dev

    side = torch.cuda.Stream(device=DEV)
    Mx, Nx = 48, 131072
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, Mx, Nx, rr.RR_F32)["ws_bytes"] > 0
    x_np = synth.normal(Mx, Nx, sigma=2.0)
    x = torch.from_numpy(x_np).to(DEV)
    torch.cuda.synchronize()
    busy = torch.randn(4096, 4096, device=DEV)
    for _ in range(4):
        busy = busy @ busy  # keeps the current stream busy meanwhile
        busy /= busy.norm()
    outs = [rr.rr_softmax_fwd(x, stream=side) for _ in range(3)]
    outs.append(rr.rr_softmax_fwd(x, stream=side.cuda_stream))  # raw handle
    side.synchronize()
    torch.cuda.synchronize()
    ref = oracle.softmax(x_np[:8])
    for y in outs:
        got = from_dev(y)
        assert np.all(np.abs(got[:8] - ref) <= 1e-5 * ref + 1e-37)
        assert torch.equal(y, outs[0])
