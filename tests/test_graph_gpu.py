"""The library's calls can be captured in a HIP graph and replayed.

The kernels allocate nothing, record no memset (the split-row workspace is left
zero by every launch that completes, exchange slots included), and
launch with ordinary kernel nodes, so a captured call replays like an eager one.
Each replay here is compared with the eager result, with eager work (new inputs
copied in) between the replays, as HIP graphs that record memset nodes have given
wrong results on replays after the first on this GPU."""
import numpy as np
import pytest
import torch

import memory_bound_row_softmax_amd as rr
import synth
from _gpu import DEV, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, M, N, dtype):
    return to_dev(synth.normal(M, N, sigma=2.0, dtype=dtype, seed=seed), dtype)


@pytest.mark.parametrize("op,dtype,M,N", [
    ("softmax", "f32", 64, 131072),     # split rows, 4 workgroups per row
    ("softmax", "bf16", 300, 4096),     # block kernel
    ("rmsnorm", "bf16", 40, 262144),    # packed, split rows
    ("xent_grad", "f32", 50, 200000),   # fused gradient, deferred exchange
    ("softmax_bwd", "f32", 64, 131072),
    ("rmsnorm_bwd", "bf16", 512, 4096),  # persistent kernel + dw pass
    ("softmax", "f32", 4, 3_000_000),   # two-pass long rows
])
def test_captured_calls_replay_like_eager_ones(op, dtype, M, N):
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    opcode = {"softmax": rr.RR_OP_SOFTMAX, "rmsnorm": rr.RR_OP_RMSNORM,
              "xent_grad": rr.RR_OP_XENT_GRAD, "softmax_bwd": rr.RR_OP_SOFTMAX_BWD,
              "rmsnorm_bwd": rr.RR_OP_RMSNORM_BWD}[op]
    x = _inputs(1, M, N, dtype)
    x2 = _inputs(2, M, N, dtype)  # a second input, copied in between replays
    w = to_dev(synth.uniform(1, N, lo=0.5, hi=1.5, dtype=dtype).reshape(N), dtype)
    lab = torch.from_numpy(synth.labels(M, N)).to(DEV)
    dloss = torch.full((M,), 0.5, dtype=torch.float32, device=DEV)
    rstd = torch.rand(M, device=DEV) + 0.5
    ws = rr.workspace(opcode, M, N, code, DEV)
    outs = {}

    def call():
        if op == "softmax":
            outs["y"] = rr.rr_softmax_fwd(x, outs.get("y"), ws=ws)
        elif op == "rmsnorm":
            outs["y"] = rr.rr_rmsnorm_fwd(x, w, 1e-6, y=outs.get("y"), ws=ws)
        elif op == "xent_grad":
            r = rr.rr_cross_entropy_fwd_bwd(x, lab, dloss, dlogits=outs.get("y"),
                                            loss=outs.get("loss"), lse=outs.get("lse"), ws=ws)
            outs["loss"], outs["lse"], outs["y"] = r
        elif op == "softmax_bwd":
            outs["y"] = rr.rr_softmax_bwd(x, x2, dx=outs.get("y"), ws=ws)
        else:
            dx, dw = rr.rr_rmsnorm_bwd(x, w, x2, rstd, dx=outs.get("y"), dw=outs.get("dw"), ws=ws)
            outs["y"], outs["dw"] = dx, dw

    # eager reference for both inputs (outputs allocated here, reused by the graph)
    call()
    torch.cuda.synchronize()
    ref1 = {k: v.clone() for k, v in outs.items()}
    saved = x.clone()
    x.copy_(x2)
    call()
    torch.cuda.synchronize()
    ref2 = {k: v.clone() for k, v in outs.items()}
    x.copy_(saved)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for i in range(4):
        second = i % 2 == 1
        x.copy_(x2 if second else saved)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = ref2 if second else ref1
        for k, v in ref.items():
            assert torch.equal(outs[k], v), f"{op} replay {i}: {k} differs from eager"
        if ws is not None:
            assert rr.rr_workspace_check(ws) == rr.RR_OK
            assert int(ws.count_nonzero()) == 0 or op == "rmsnorm_bwd"
