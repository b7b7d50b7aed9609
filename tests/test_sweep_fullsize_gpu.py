"""Parity at every point of the 3-op x 2-dtype sweep (M in {8192, 16384, 32768}, N in
{256 .. 262144}) at its full size, with the plan the bench times.

As in the bench's sweep, the first 128 rows of a workload are generated on the host
and repeated down the matrix, so that the largest points (32 GiB of input) are
built in seconds.  Every row of the output is then the result of one of those 128
input rows: a spread of rows across the matrix is checked element by element
against the oracle, and softmax rows must sum to 1 (cross-entropy: loss = lse -
x[label], max <= lse <= max + ln N) on every row."""
import math

import numpy as np
import pytest
import torch

import memory_bound_row_softmax_amd as rr
import oracle
from synth import workloads as W
from _gpu import DEV, check_out, from_dev, record, say, to_dev
from _verify import Stats, check_f32, check_rows_device

pytestmark = pytest.mark.gpu

HOST_ROWS = 128


def _rows(M):
    return np.unique(np.concatenate([[0, 1, M // 2, M - 1], np.linspace(0, M - 1, 8)])
                     .astype(np.int64))


@pytest.mark.parametrize("w", W.sweep(), ids=lambda w: w.name)
def test_sweep_point_at_full_size(w):
    say("sweep full size", w.name)
    x_np = W.x_rows(w, nrows=HOST_ROWS)
    x = to_dev(x_np, w.dtype).repeat(w.M // HOST_ROWS, 1)
    rows = _rows(w.M)
    rows_t = torch.from_numpy(rows).to(DEV)
    src = x_np[rows % HOST_ROWS]
    code = rr.RR_F32 if w.dtype == "f32" else rr.RR_BF16
    if w.op == "xent":
        lab_np = W.label_rows(w)
        lab = torch.from_numpy(lab_np).to(DEV)
        loss, lse = rr.rr_cross_entropy_fwd(x, lab)
        torch.cuda.synchronize()
        ref_loss, ref_lse = oracle.cross_entropy(src, lab_np[rows])
        record(w.name + f" lse ({rows.size} rows)",
               check_f32(lse[rows_t].cpu().numpy(), ref_lse, w.name + " lse"))
        record(w.name + f" loss ({rows.size} rows)",
               check_f32(loss[rows_t].cpu().numpy(), ref_loss, w.name + " loss"))
        for r0 in range(0, w.M, 4096):
            xs = x[r0:r0 + 4096]
            mx = xs.max(dim=1).values.double()
            l = lse[r0:r0 + 4096].double()
            assert bool(((l >= mx - 1e-5 * mx.abs()) & (l <= mx + math.log(w.N) + 1e-4)).all())
            xl = xs.gather(1, lab[r0:r0 + 4096].long()[:, None])[:, 0].double()
            err = (loss[r0:r0 + 4096].double() - (l - xl)).abs().max()
            assert float(err) <= 4e-6 * max(1.0, float(l.abs().max()))
        return
    ws = rr.workspace(rr.RR_OP_SOFTMAX if w.op == "softmax" else rr.RR_OP_RMSNORM, w.M, w.N,
                      code, DEV)
    if w.op == "softmax":
        y = rr.rr_softmax_fwd(x, ws=ws)
        ref = oracle.softmax(src)
    else:
        w_np = W.weight(w)
        y = rr.rr_rmsnorm_fwd(x, to_dev(w_np, w.dtype), w.eps, ws=ws)
        ref = oracle.rmsnorm(src, w_np, w.eps)
    torch.cuda.synchronize()
    if ws is not None:
        assert rr.rr_workspace_check(ws) == rr.RR_OK
    record(w.name + f" ({rows.size} rows)", check_out(from_dev(y[rows_t]), ref, w.dtype, w.name))
    if w.op == "softmax":
        step = max(1, (1 << 26) // w.N)
        for r0 in range(0, w.M, step):
            s = y[r0:r0 + step].double().sum(dim=1)
            assert float((s - 1.0).abs().max()) < (1e-4 if w.dtype == "f32" else 2e-2), r0


# Rows whose length is not a power of two, at full size with the bench's plan: a
# 151936-entry vocabulary (softmax) and 200000-wide rows (RMSNorm).  The members of
# a split row hold interleaved 4 KiB granules (RMSNorm fp32 on 8 workgroups and bf16
# packed on 8 of 256 lanes) or one contiguous part each (softmax fp32 and bf16 on exactly 5, the
# last part shorter).
UNEVEN = W.UNEVEN
UNEVEN_G = {"softmax_f32": 5, "softmax_bf16": 5, "rmsnorm_f32": 8, "rmsnorm_bf16": 8}


@pytest.mark.parametrize("w", UNEVEN, ids=lambda w: w.name)
def test_uneven_rows_at_full_size(w):
    code = rr.RR_F32 if w.dtype == "f32" else rr.RR_BF16
    op = rr.RR_OP_SOFTMAX if w.op == "softmax" else rr.RR_OP_RMSNORM
    p = rr.rr_plan_query(op, w.M, w.N, code)
    assert p["path"] == 1 and p["groups_per_row"] == UNEVEN_G[f"{w.op}_{w.dtype}"], p
    say("uneven full size", w.name)
    x_np = W.x_rows(w, nrows=HOST_ROWS)
    x = to_dev(x_np, w.dtype).repeat(w.M // HOST_ROWS, 1)
    rows = _rows(w.M)
    rows_t = torch.from_numpy(rows).to(DEV)
    src = x_np[rows % HOST_ROWS]
    ws = rr.workspace(op, w.M, w.N, code, DEV)
    if w.op == "softmax":
        y = rr.rr_softmax_fwd(x, ws=ws)
        ref = oracle.softmax(src)
    else:
        w_np = W.weight(w)
        y = rr.rr_rmsnorm_fwd(x, to_dev(w_np, w.dtype), w.eps, ws=ws)
        ref = oracle.rmsnorm(src, w_np, w.eps)
    torch.cuda.synchronize()
    assert rr.rr_workspace_check(ws) == rr.RR_OK
    assert int(ws.count_nonzero()) == 0
    check_out(from_dev(y[rows_t]), ref, w.dtype, w.name)
    # Every row against the oracle's result for its host row (rows repeat every
    # HOST_ROWS), on the device: fp32 within 1e-5 relative, bf16 within one ulp.
    if w.op == "softmax":
        full = oracle.softmax(x_np)
    else:
        full = oracle.rmsnorm(x_np, w_np, w.eps)
    ref_t = torch.from_numpy(np.ascontiguousarray(full, dtype=np.float64)).to(DEV)
    stats = Stats(w.dtype)
    worst_rep = 0.0
    for r0 in range(0, w.M, HOST_ROWS):
        blk = y[r0:r0 + HOST_ROWS]
        check_rows_device(blk, ref_t, w.dtype, stats, f"{w.name} rows {r0}..")
        worst_rep = max(worst_rep, float((blk.double() - y[:HOST_ROWS].double()).abs().max()))
    record(w.name + " (all rows)", stats)
    say("largest difference between repeats of a row:", worst_rep)
