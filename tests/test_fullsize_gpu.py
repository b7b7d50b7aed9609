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


@pytest.mark.parametrize("w", [w for w in W.BACKWARD if w.op == "xent_grad"], ids=lambda w: w.name)
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


def _bwd_workload(op):
    return [w for w in W.BACKWARD if w.op == op]


@pytest.mark.parametrize("w", _bwd_workload("softmax_bwd"), ids=lambda w: w.name)
def test_softmax_bwd_fullsize_sampled(w):
    """Softmax backward at its benchmarked shapes; y is the oracle's softmax of the
    workload's x on sampled rows (and the library's forward on the rest, whose rows
    are only checked for sum(dx) = (1 - sum y) * c)."""
    from _gpu import softmax_bwd_scale
    from _verify import check_grad

    say("full-size", w.name, "generate")
    x_np = W.x_rows(w)
    dy_np = W.dy_rows(w)
    code = rr.RR_F32 if w.dtype == "f32" else rr.RR_BF16
    y = rr.rr_softmax_fwd(to_dev(x_np, w.dtype))
    rows = _sample_rows(w.M, 32)
    y64 = oracle.softmax(x_np[rows]).astype(np.float32)
    y_rows = y64 if w.dtype == "f32" else synth.f32_to_bf16(y64)
    y[torch.from_numpy(rows).to(DEV)] = to_dev(y_rows, w.dtype)
    dy = to_dev(dy_np, w.dtype)
    ws = rr.workspace(rr.RR_OP_SOFTMAX_BWD, w.M, w.N, code, DEV)
    say("full-size", w.name, "run")
    dx = rr.rr_softmax_bwd(y, dy, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.softmax_backward(y_rows, dy_np[rows])
    check_grad(from_dev(dx[torch.from_numpy(rows).to(DEV)]), ref,
               softmax_bwd_scale(y_rows, dy_np[rows], w.dtype), w.dtype, "dx sampled")
    del x_np, dy_np
    for r0 in range(0, w.M, 2048):
        yy, dd, xx = (t[r0:r0 + 2048].double() for t in (y, dy, dx))
        c = (yy * dd).sum(dim=1)
        want = (1.0 - yy.sum(dim=1)) * c
        scale = (yy * dd.abs()).sum(dim=1) + c.abs()
        got = xx.sum(dim=1)
        tol = 1e-4 if w.dtype == "f32" else 5e-2
        assert bool(((got - want).abs() <= tol * scale + 1e-6).all()), r0


@pytest.mark.parametrize("w", _bwd_workload("rmsnorm_bwd"), ids=lambda w: w.name)
def test_rmsnorm_bwd_fullsize(w):
    """RMSNorm backward at its benchmarked shapes: dx on sampled rows and dw on every
    column against the oracle (rstd from the oracle's forward, rounded to fp32)."""
    from _gpu import rmsnorm_bwd_scales
    from _verify import check_grad

    say("full-size", w.name, "generate")
    x_np, w_np, dy_np = W.x_rows(w), W.weight(w), W.dy_rows(w)
    _, r64 = oracle.rmsnorm(x_np, w_np, w.eps, want_rstd=True)
    r_np = r64.astype(np.float32)
    code = rr.RR_F32 if w.dtype == "f32" else rr.RR_BF16
    ws = rr.workspace(rr.RR_OP_RMSNORM_BWD, w.M, w.N, code, DEV)
    say("full-size", w.name, "run")
    dx, dw = rr.rr_rmsnorm_bwd(to_dev(x_np, w.dtype), to_dev(w_np, w.dtype), to_dev(dy_np, w.dtype),
                               torch.from_numpy(r_np).to(DEV), ws=ws)
    torch.cuda.synchronize()
    rows = _sample_rows(w.M, 32)
    ref_dx, _ = oracle.rmsnorm_backward(x_np[rows], w_np, dy_np[rows], r_np[rows])
    sdx, _ = rmsnorm_bwd_scales(x_np[rows], w_np, dy_np[rows], r_np[rows], w.dtype)
    check_grad(from_dev(dx[torch.from_numpy(rows).to(DEV)]), ref_dx, sdx, w.dtype, "dx sampled")
    _, ref_dw = oracle.rmsnorm_backward(x_np, w_np, dy_np, r_np)
    _, sdw = rmsnorm_bwd_scales(x_np, w_np, dy_np, r_np, w.dtype)
    check_grad(dw.cpu().numpy(), ref_dw, sdw, "f32", "dw all columns")
