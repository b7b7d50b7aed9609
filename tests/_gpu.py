"""Helpers of the GPU tests: move seeded numpy inputs to the device, run an op
through the C ABI, bring the outputs back, and compare them with the oracle."""
from __future__ import annotations

import sys
from contextlib import contextmanager

import numpy as np
import torch

import memory_bound_row_softmax_amd as rr
import oracle
from _verify import check_bf16, check_f32, check_grad

DEV = "cuda:0"


def say(*a):
    """Names the case about to run on the GPU, flushed before the GPU step."""
    print("[gpu]", *a, file=sys.stderr, flush=True)


def record(config: str, stats, **extra):
    """Prints one accuracy line for a configuration, and appends it as JSON to the
    file RR_PARITY_LOG names (if set); conftest.py turns that file into a table."""
    import json
    import os

    d = {"config": config, **stats.as_dict(), **extra}
    print("[parity]", json.dumps(d), file=sys.stderr, flush=True)
    path = os.environ.get("RR_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(d) + "\n")
    return stats


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def from_dev(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@contextmanager
def forced(P=None, R=None, G=None, spin=None, kind=None, groups=None):
    """Test-only plan and launch overrides (rr_set_test_overrides), restored after."""
    rr.set_test_overrides(kind=kind, P=P, R=R, G=G, groups=groups, spin=spin)
    try:
        yield
    finally:
        rr.set_test_overrides()


def check_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    if dtype == "f32":
        return check_f32(got, ref, what)
    return check_bf16(got, ref, what)


def run_softmax(x_np, dtype, ws=None, inplace=False):
    x = to_dev(x_np, dtype)
    y = x if inplace else torch.empty_like(x)
    rr.rr_softmax_fwd(x, y, ws=ws)
    torch.cuda.synchronize()
    return from_dev(y)


def run_rmsnorm(x_np, w_np, eps, dtype, want_rstd=False):
    x = to_dev(x_np, dtype)
    w = to_dev(w_np, dtype)
    rstd = torch.empty(x.shape[0], dtype=torch.float32, device=DEV) if want_rstd else None
    y = rr.rr_rmsnorm_fwd(x, w, eps, rstd=rstd)
    torch.cuda.synchronize()
    return (from_dev(y), rstd.cpu().numpy()) if want_rstd else from_dev(y)


def run_xent(x_np, labels_np, dtype):
    x = to_dev(x_np, dtype)
    lab = torch.from_numpy(np.ascontiguousarray(labels_np, dtype=np.int32)).to(DEV)
    loss, lse = rr.rr_cross_entropy_fwd(x, lab)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), lse.cpu().numpy()


def parity_softmax(x_np, dtype, what):
    got = run_softmax(x_np, dtype)
    return check_out(got, oracle.softmax(x_np), dtype, what)


def parity_rmsnorm(x_np, w_np, eps, dtype, what):
    got, rstd = run_rmsnorm(x_np, w_np, eps, dtype, want_rstd=True)
    ref, ref_rstd = oracle.rmsnorm(x_np, w_np, eps, want_rstd=True)
    check_f32(rstd, ref_rstd, what + " rstd")
    return check_out(got, ref, dtype, what)


def parity_xent(x_np, labels_np, dtype, what):
    loss, lse = run_xent(x_np, labels_np, dtype)
    ref_loss, ref_lse = oracle.cross_entropy(x_np, labels_np)
    check_f32(lse, ref_lse, what + " lse")
    return check_f32(loss, ref_loss, what + " loss")


def run_xent_grad(x_np, labels_np, dloss_np, dtype, inplace=False):
    x = to_dev(x_np, dtype)
    lab = torch.from_numpy(np.ascontiguousarray(labels_np, dtype=np.int32)).to(DEV)
    g = torch.from_numpy(np.ascontiguousarray(dloss_np, dtype=np.float32)).to(DEV)
    loss, lse, dx = rr.rr_cross_entropy_fwd_bwd(x, lab, g, dlogits=x if inplace else None)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), lse.cpu().numpy(), from_dev(dx)


def xent_grad_scale(x_np, labels_np, dloss_np):
    """Per-element size of the gradient's terms: (p + onehot) * |dloss|."""
    p = oracle.softmax(x_np)
    M, N = p.shape
    lab = np.asarray(labels_np)
    ok = (lab >= 0) & (lab < N)
    p[np.flatnonzero(ok), lab[ok]] += 1.0
    return p * np.abs(np.asarray(dloss_np, dtype=np.float64))[:, None]


def parity_xent_grad(x_np, labels_np, dloss_np, dtype, what, inplace=False):
    loss, lse, dx = run_xent_grad(x_np, labels_np, dloss_np, dtype, inplace=inplace)
    ref_loss, ref_lse, ref_dx = oracle.cross_entropy_grad(x_np, labels_np, dloss_np)
    check_f32(lse, ref_lse, what + " lse")
    check_f32(loss, ref_loss, what + " loss")
    return check_grad(dx, ref_dx, xent_grad_scale(x_np, labels_np, dloss_np), dtype, what + " dx")


def softmax_bwd_inputs(M, N, dtype, sigma=2.0):
    """y = the softmax of a seeded row (oracle, rounded to the dtype), dy ~ N(0, 1)."""
    import synth

    y64 = oracle.softmax(synth.normal(M, N, sigma=sigma))
    y = y64.astype(np.float32) if dtype == "f32" else synth.f32_to_bf16(y64.astype(np.float32))
    dy = synth.normal(M, N, dtype=dtype, stream=synth.STREAM_DY)
    return y, dy


def _dec(a, dtype):
    return (a.astype(np.float64) if dtype == "f32"
            else (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def softmax_bwd_scale(y_np, dy_np, dtype):
    y, dy = _dec(y_np, dtype), _dec(dy_np, dtype)
    return np.abs(y) * (np.abs(dy) + np.abs(y * dy).sum(axis=1, keepdims=True))


def parity_softmax_bwd(y_np, dy_np, dtype, what, inplace=None):
    y, dy = to_dev(y_np, dtype), to_dev(dy_np, dtype)
    dx = {"y": y, "dy": dy}.get(inplace)
    dx = rr.rr_softmax_bwd(y, dy, dx=dx)
    torch.cuda.synchronize()
    ref = oracle.softmax_backward(y_np, dy_np)
    return check_grad(from_dev(dx), ref, softmax_bwd_scale(y_np, dy_np, dtype), dtype, what)


def rmsnorm_bwd_inputs(M, N, dtype, eps=1e-6):
    """x ~ N(0, 1), w ~ U(0.5, 1.5), dy ~ N(0, 1) in the dtype; rstd is the forward's
    r of each row (oracle, rounded to fp32)."""
    import synth

    x = synth.normal(M, N, dtype=dtype)
    w = synth.uniform(1, N, lo=0.5, hi=1.5, dtype=dtype).reshape(N)
    dy = synth.normal(M, N, dtype=dtype, stream=synth.STREAM_DY)
    _, r = oracle.rmsnorm(x, w, eps, want_rstd=True)
    return x, w, dy, r.astype(np.float32)


def rmsnorm_bwd_scales(x_np, w_np, dy_np, rstd, dtype):
    """Per-element sizes of the terms of dx, and per-column of dw."""
    x, w, dy = _dec(x_np, dtype), _dec(w_np, dtype), _dec(dy_np, dtype)
    r = rstd.astype(np.float64)[:, None]
    N = x.shape[1]
    cabs = np.abs(dy * w[None, :] * x).sum(axis=1, keepdims=True)
    sdx = r * np.abs(w[None, :] * dy) + r ** 3 * np.abs(x) * cabs / N
    sdw = np.abs(dy * x * r).sum(axis=0)
    return sdx, sdw


def parity_rmsnorm_bwd(x_np, w_np, dy_np, rstd, dtype, what, inplace=None, ws=None):
    x, w, dy = to_dev(x_np, dtype), to_dev(w_np, dtype), to_dev(dy_np, dtype)
    r = torch.from_numpy(np.ascontiguousarray(rstd, dtype=np.float32)).to(DEV)
    dx = {"x": x, "dy": dy}.get(inplace)
    dx, dw = rr.rr_rmsnorm_bwd(x, w, dy, r, dx=dx, ws=ws)
    torch.cuda.synchronize()
    ref_dx, ref_dw = oracle.rmsnorm_backward(x_np, w_np, dy_np, rstd)
    sdx, sdw = rmsnorm_bwd_scales(x_np, w_np, dy_np, rstd, dtype)
    check_grad(from_dev(dx), ref_dx, sdx, dtype, what + " dx")
    check_grad(dw.cpu().numpy(), ref_dw, sdw, "f32", what + " dw")
    return dx, dw
