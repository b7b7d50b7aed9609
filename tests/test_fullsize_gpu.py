"""Parity at the benchmarked sizes, in the launch configuration the bench times.

The oracle checks a spread of sampled rows element by element (it cannot do all
rows in seconds); properties that hold at any size are checked on every row:
softmax rows sum to 1, and max(x) <= lse <= max(x) + ln N and
loss = lse - x[label] for cross-entropy.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W
from _gpu import DEV, check_out, from_dev, say, to_dev
from _verify import check_f32

import memory_bound_row_softmax_amd as rr

pytestmark = pytest.mark.gpu


def _sample_rows(M, k=64):
    rows = np.unique(np.linspace(0, M - 1, k).astype(np.int64))
    return rows


def test_rmsnorm_bf16_16384x4096_all_rows():
    w = W.RMSNORM_MAIN
    say("full-size", w.name, "generate")
    x_np = W.x_rows(w)
    w_np = W.weight(w)
    x, wt = to_dev(x_np, w.dtype), to_dev(w_np, w.dtype)
    say("full-size", w.name, "run")
    y = rr.rr_rmsnorm_fwd(x, wt, w.eps)
    torch.cuda.synchronize()
    check_out(from_dev(y), oracle.rmsnorm(x_np, w_np, w.eps), w.dtype, w.name)


def test_xent_f32_8192x131072_sampled():
    w = W.XENT_VOCAB
    say("full-size", w.name, "generate")
    x_np = W.x_rows(w)
    lab_np = W.label_rows(w)
    x = to_dev(x_np, w.dtype)
    lab = torch.from_numpy(lab_np).to(DEV)
    say("full-size", w.name, "run")
    loss, lse = rr.rr_cross_entropy_fwd(x, lab)
    torch.cuda.synchronize()
    rows = _sample_rows(w.M)
    ref_loss, ref_lse = oracle.cross_entropy(x_np[rows], lab_np[rows])
    check_f32(lse.cpu().numpy()[rows], ref_lse, "lse sampled")
    check_f32(loss.cpu().numpy()[rows], ref_loss, "loss sampled")
    # every row
    mx = x.max(dim=1).values.double()
    l = lse.double()
    assert bool(((l >= mx - 1e-5 * mx.abs()) & (l <= mx + math.log(w.N) + 1e-4)).all())
    xl = x.gather(1, lab.long()[:, None])[:, 0].double()
    assert float((loss.double() - (l - xl)).abs().max()) <= 4e-6 * float(l.abs().max())


def test_softmax_f32_16384x131072_spiky_sampled():
    w = W.SOFTMAX_SPIKY
    say("full-size", w.name, "generate")
    x_np = W.x_rows(w)
    x = to_dev(x_np, w.dtype)
    y = torch.empty_like(x)
    ws = rr.workspace(rr.RR_OP_SOFTMAX, w.M, w.N, rr.RR_F32, DEV)
    say("full-size", w.name, "run")
    rr.rr_softmax_fwd(x, y, ws=ws)
    torch.cuda.synchronize()
    assert rr.rr_workspace_check(ws) == rr.RR_OK
    rows = _sample_rows(w.M)
    check_out(y[torch.from_numpy(rows).to(DEV)].cpu().numpy(), oracle.softmax(x_np[rows]),
              w.dtype, "softmax spiky sampled")
    del x_np
    for r0 in range(0, w.M, 2048):
        s = y[r0:r0 + 2048].double().sum(dim=1)
        assert float((s - 1.0).abs().max()) < 1e-5, r0


@pytest.mark.parametrize("w", W.BACKWARD, ids=lambda w: w.name)
def test_xent_grad_fullsize_sampled(w):
    """The fused cross-entropy gradient at its benchmarked shapes: sampled rows
    against the oracle, and on every row the gradient sums to zero and loss
    equals lse - x[label]."""
    from _gpu import xent_grad_scale
    from _verify import check_grad

    say("full-size", w.name, "generate")
    x_np = W.x_rows(w)
    lab_np = W.label_rows(w)
    g_np = W.dloss_rows(w)
    x = to_dev(x_np, w.dtype)
    lab = torch.from_numpy(lab_np).to(DEV)
    g = torch.from_numpy(g_np).to(DEV)
    code = rr.RR_F32 if w.dtype == "f32" else rr.RR_BF16
    ws = rr.workspace(rr.RR_OP_XENT_GRAD, w.M, w.N, code, DEV)
    say("full-size", w.name, "run")
    loss, lse, dx = rr.rr_cross_entropy_fwd_bwd(x, lab, g, ws=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert rr.rr_workspace_check(ws) == rr.RR_OK
    rows = _sample_rows(w.M, 32)
    ref_loss, ref_lse, ref_dx = oracle.cross_entropy_grad(x_np[rows], lab_np[rows], g_np[rows])
    check_f32(lse.cpu().numpy()[rows], ref_lse, "lse sampled")
    check_f32(loss.cpu().numpy()[rows], ref_loss, "loss sampled")
    got = from_dev(dx[torch.from_numpy(rows).to(DEV)])
    check_grad(got, ref_dx, xent_grad_scale(x_np[rows], lab_np[rows], g_np[rows]), w.dtype,
               "dx sampled")
    del x_np
    xl = x.gather(1, lab.long()[:, None])[:, 0].double()
    assert float((loss.double() - (lse.double() - xl)).abs().max()) <= 4e-6 * float(lse.abs().max())
    tol = 1e-4 if w.dtype == "f32" else 0.05
    for r0 in range(0, w.M, 2048):
        s = dx[r0:r0 + 2048].double().sum(dim=1)
        assert float(s.abs().max()) < tol, r0
