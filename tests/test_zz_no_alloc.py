"""rr_softmax_fwd_static, the softmax forward that allocates nothing (rows split over
several workgroups exchange through a device array the library holds on each GPU),
against rr_softmax_fwd with a workspace the caller allocates: the same bits, called
through the C ABI, on two calls in a row (the second with a smaller input, so the
array holds the first call's leftovers), for split rows (the exchange inside a row's
step, and deferred, up to 256 workgroups per row), rows read twice, and a plan that
needs no workspace."""
import pytest
import torch

import memory_bound_row_softmax_amd as rr
import synth
from _gpu import DEV, say, to_dev

pytestmark = pytest.mark.gpu

# (M, N) pairs: the second call of each pair is smaller than the first
PAIRS = [
    ((64, 262144), (16, 70000)),      # 8 then 4 workgroups per row (deferred, then not)
    ((200, 131072), (7, 131072)),     # 4 per row, fewer rows
    ((8, 5_000_000), (3, 3_000_000)),  # rows read twice (64 then 32 per row)
    ((3, 8_388_608), (2, 8_000_000)),  # 256 workgroups per row, one on every CU
    ((256, 1024), (100, 1000)),       # no workspace at all
]


def _one(dtype, M, N):
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    x = to_dev(synth.normal(M, N, sigma=2.0, dtype=dtype), dtype)
    ws = rr.workspace(rr.RR_OP_SOFTMAX, M, N, code, DEV)
    y_ref = torch.empty_like(x)
    sp = torch.cuda.current_stream().cuda_stream
    assert rr.softmax_fwd_raw(x.data_ptr(), y_ref.data_ptr(), M, N, code,
                              ws.data_ptr() if ws is not None else 0,
                              ws.numel() if ws is not None else 0, sp) == rr.RR_OK
    y = torch.full_like(x, float("nan"))
    assert rr.softmax_fwd_static_raw(x.data_ptr(), y.data_ptr(), M, N, code, sp) == rr.RR_OK
    torch.cuda.synchronize()
    if ws is not None:
        assert rr.rr_workspace_check(ws) == rr.RR_OK
    assert torch.equal(y, y_ref), f"{dtype} {M}x{N}: static workspace differs"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}x{p[0][1]}")
def test_no_alloc_softmax_matches_caller_workspace(pair, dtype):
    if dtype == "bf16" and pair[0][1] == 5_000_000:
        # bf16 rows that fill less than 9/10 of 64 or 128 workgroups read twice
        pair = ((8, 2_500_000), (3, 1_500_000))
    for M, N in pair:
        say("no-alloc softmax", dtype, M, N)
        _one(dtype, M, N)


def test_no_alloc_softmax_rejects_bad_arguments():
    x = torch.zeros(4, 8, device=DEV)
    sp = torch.cuda.current_stream().cuda_stream
    assert rr.softmax_fwd_static_raw(0, x.data_ptr(), 4, 8, rr.RR_F32, sp) == \
        rr.RR_ERR_INVALID_ARGUMENT
    assert rr.softmax_fwd_static_raw(x.data_ptr(), x.data_ptr(), 4, 8, 7, sp) == \
        rr.RR_ERR_INVALID_ARGUMENT
    assert rr.softmax_fwd_static_raw(x.data_ptr(), x.data_ptr(), 0, 8, rr.RR_F32, sp) == rr.RR_OK
