"""GPU parity of the backward passes: the HIP kernels (through the C ABI) against
the double-precision oracle, element by element, on seeded inputs.

RMSNorm backward: dx and dw from x, w, dy and the forward's rstd (the oracle's,
rounded to fp32); dx within the bound with scale r|w_j dy_j| + r^3 |x_j|
sum_k |dy_k w_k x_k| / N, dw (fp32, summed over the rows through per-workgroup
partial rows) within relative 1e-5 of sum_i |dy_ij x_ij r_i|.

Softmax backward: dx from the forward output y (the oracle's softmax of a seeded
row, rounded to the dtype) and dy ~ N(0, 1), within the cancellation-aware bound
with scale y_j * (|dy_j| + sum_k |y_k dy_k|).

Cross-entropy forward fused with its gradient: loss and lse within relative 1e-5,
the gradient within the cancellation-aware bound of tests/_verify.py.  The fused
kernel is the softmax kernel with another epilogue, so every softmax path (lane
group, workgroup, persistent stream, split rows, per-element) is run.
"""
import numpy as np
import pytest
import torch

import memory_bound_row_softmax_amd as rr
import oracle
import synth
from _gpu import (DEV, forced, from_dev, parity_rmsnorm_bwd, parity_softmax_bwd, parity_xent_grad,
                  rmsnorm_bwd_inputs, rmsnorm_bwd_scales, run_xent_grad, say, softmax_bwd_inputs,
                  softmax_bwd_scale, to_dev, xent_grad_scale)
from _verify import check_f32, check_grad

pytestmark = pytest.mark.gpu

# launches of a determinism test, each compared with the first bit for bit
REPEATS = 20

DTYPES = ("f32", "bf16")
SHAPES = [(256, 1024), (64, 1), (64, 3), (70, 255), (33, 257), (37, 1000), (16, 4095),
          (16, 4096), (9, 4097), (8, 16384), (5, 20000), (4, 65536), (3, 65537), (3, 131072),
          (2, 200000), (2, 262144)]


def _dloss(M, row0=0):
    return synth.uniform(1, M, lo=0.5, hi=1.5, stream=synth.STREAM_DLOSS, row0=row0)[0]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", SHAPES)
def test_xent_grad(M, N, dtype):
    say("xent grad", dtype, M, N)
    x = synth.normal(M, N, sigma=2.0, dtype=dtype)
    parity_xent_grad(x, synth.labels(M, N), _dloss(M), dtype, f"xent grad {dtype} {M}x{N}")


@pytest.mark.parametrize("N,G", [(40000, 3), (70000, 5), (90000, 6), (100000, 7),
                                 (140000, 9), (151936, 10), (180000, 11), (196608, 12),
                                 (200000, 13), (220000, 14), (240000, 15)])
def test_xent_grad_bf16_exact_groups(N, G):
    """bf16 rows of 32769 to 262144 elements: split over exactly ceil(N / 16384)
    workgroups of 64 values x 256 lanes (the plan at 16384 rows; 50 rows run)."""
    M = 50
    p = rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 16384, N, rr.RR_BF16)
    assert (p["path"], p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]) == (1, 64, 256, G)
    say("xent grad exact groups", G, M, N)
    x = synth.normal(M, N, sigma=2.0, dtype="bf16")
    with forced(64, 256, G, kind="stream"):
        parity_xent_grad(x, synth.labels(M, N), _dloss(M), "bf16", f"xent grad bf16 G={G} {M}x{N}")


FORCED = [("stream", 64, 256, 2, 300, 20000), ("stream", 32, 512, 16, 97, 70000),
          ("stream", 64, 512, 2, 50, 65536), ("stream", 64, 512, 16, 9, 500000),
          ("stream", 16, 1024, 1, 700, 16000), ("stream", 32, 512, 1, 3, 16384),
          ("stream", 16, 1024, 8, 200, 100000), ("block", 16, 16, 1, 100, 256),
          ("block", 32, 128, 1, 31, 4000), ("block", 16, 1024, 1, 5, 16384),
          ("block", 64, 1024, 1, 6, 65536), ("stream", 64, 512, 32, 5, 1_000_000),
          # bf16 on 64 x 256 lanes rewrites the label's element after the row's
          # stores: 1, 2, 4, 8, 10 and 16 workgroups, labels in every member
          ("stream", 64, 256, 1, 400, 16000), ("stream", 64, 256, 4, 120, 60000),
          ("stream", 64, 256, 8, 80, 131072), ("stream", 64, 256, 10, 60, 151936),
          ("stream", 64, 256, 16, 40, 250000), ("stream", 32, 512, 2, 200, 30000)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind,P,R,G,M,N", FORCED)
def test_xent_grad_forced_plans(kind, P, R, G, M, N, dtype):
    with forced(P, R, G, kind=kind):
        try:
            rr.rr_plan_query(rr.RR_OP_XENT_GRAD, M, N, rr.RR_F32 if dtype == "f32" else rr.RR_BF16)
        except rr.RRError:
            pytest.skip("not compiled for this dtype (register budget)")
        say("xent grad forced", kind, P, R, G, dtype, M, N)
        x = synth.normal(M, N, sigma=2.0, dtype=dtype)
        parity_xent_grad(x, synth.labels(M, N), _dloss(M), dtype, f"xent grad {kind} {P},{R},{G}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", [(64, 1024), (8, 131072)])
def test_xent_grad_in_place(M, N, dtype):
    say("xent grad in place", dtype, M, N)
    x = synth.normal(M, N, sigma=2.0, dtype=dtype)
    parity_xent_grad(x, synth.labels(M, N), _dloss(M), dtype, "in-place xent grad", inplace=True)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", [(2, (1 << 21) + 8), (1, 3_000_000)])
def test_xent_grad_long_rows(M, N, dtype):
    """Rows past the on-chip plans: the two-read kernel (the row's max and sum over a
    first read, dlogits from a second), also in place (x[label] is read before any
    workgroup of the row writes)."""
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    assert rr.rr_plan_query(rr.RR_OP_XENT_GRAD, M, N, code)["path"] == 4
    x = synth.normal(M, N, sigma=2.0, dtype=dtype)
    for inplace in (False, True):
        say("xent grad long", dtype, M, N, inplace)
        parity_xent_grad(x, synth.labels(M, N), _dloss(M), dtype,
                         f"xent grad long {dtype} {M}x{N}", inplace=inplace)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", [(7, 1000), (33, 40000), (5, 16 * 16384 + 5), (70, 9)])
def test_xent_grad_long_row_kernel_forced_at_short_rows(M, N, dtype):
    """The two-read kernel forced on short rows: members with no tile, ragged tails,
    labels in every position of a tile; invalid labels and constant rows."""
    with forced(kind="long"):
        say("xent grad long forced", dtype, M, N)
        x = synth.normal(M, N, sigma=2.0, dtype=dtype)
        parity_xent_grad(x, synth.labels(M, N), _dloss(M), dtype, f"xent grad long forced {M}x{N}")
        if N == 1000:
            lab = np.array([0, -1, N, N - 1, 1 << 30, 7, -(1 << 30)], dtype=np.int32)
            parity_xent_grad(x, lab, _dloss(M), dtype, "xent grad long forced, invalid labels")
            c = np.full((4, 4096), 2.5, dtype=np.float32)
            c = c if dtype == "f32" else synth.f32_to_bf16(c)
            parity_xent_grad(c, np.array([0, 5, 4095, 17], np.int32), _dloss(4), dtype,
                             "xent grad long forced, constant rows")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("N", [64, 1000, 4096, 40000, 131072, 300001])
def test_xent_grad_unaligned(N, dtype):
    M = 6
    x_np = synth.normal(M, N, sigma=2.0, dtype=dtype)
    lab, g = synth.labels(M, N), _dloss(M)
    xs = to_dev(np.concatenate([np.zeros(1, x_np.dtype), x_np.ravel()]), dtype)[1:].view(M, N)
    dx = torch.empty(M * N + 1, dtype=xs.dtype, device=DEV)[1:].view(M, N)
    assert xs.data_ptr() % 16 != 0
    say("xent grad unaligned", dtype, N)
    loss, lse, dx = rr.rr_cross_entropy_fwd_bwd(xs, torch.from_numpy(lab).to(DEV),
                                                torch.from_numpy(g).to(DEV), dlogits=dx)
    torch.cuda.synchronize()
    ref_loss, ref_lse, ref_dx = oracle.cross_entropy_grad(x_np, lab, g)
    check_f32(loss.cpu().numpy(), ref_loss, "unaligned loss")
    check_f32(lse.cpu().numpy(), ref_lse, "unaligned lse")
    check_grad(from_dev(dx), ref_dx, xent_grad_scale(x_np, lab, g), dtype, "unaligned dx")


@pytest.mark.parametrize("dtype", DTYPES)
def test_xent_grad_special_rows(dtype):
    say("xent grad special rows", dtype)
    # invalid labels: NaN loss and a NaN gradient row; valid rows untouched
    M, N = 8, 5000
    x = synth.normal(M, N, sigma=2.0, dtype=dtype)
    lab = np.array([0, -1, N, N - 1, 1 << 30, 7, -(1 << 30), 4999], dtype=np.int32)
    parity_xent_grad(x, lab, _dloss(M), dtype, "invalid labels")
    # spiky rows (many exact maxima) and large values
    x = synth.normal(40, 8192, dtype=dtype)
    synth.spikes_(x, p=0.01, value=20.0, dtype=dtype)
    parity_xent_grad(x, synth.labels(40, 8192), _dloss(40), dtype, "spiky xent grad")
    big = (synth.normal(8, 3000) * 30 + 1000.0).astype(np.float32)
    big = big if dtype == "f32" else synth.f32_to_bf16(big)
    parity_xent_grad(big, synth.labels(8, 3000), _dloss(8), dtype, "large-value xent grad")
    # N = 1: loss 0, gradient 0; constant rows: gradient (1/N - onehot) * dloss
    x = synth.normal(50, 1, sigma=5.0, dtype=dtype)
    loss, _, dx = run_xent_grad(x, np.zeros(50, np.int32), _dloss(50), dtype)
    assert np.all(loss == 0.0)
    assert np.all((dx if dtype == "f32" else (dx.astype(np.uint32) << 16).view(np.float32)) == 0.0)
    c = np.full((4, 4096), 2.5, dtype=np.float32)
    c = c if dtype == "f32" else synth.f32_to_bf16(c)
    parity_xent_grad(c, np.array([0, 5, 4095, 17], np.int32), _dloss(4), dtype, "constant rows")


def test_xent_grad_negative_and_zero_dloss():
    say("xent grad signed dloss")
    M, N = 16, 3000
    x = synth.normal(M, N, sigma=2.0)
    g = np.linspace(-2.0, 2.0, M).astype(np.float32)
    g[3] = 0.0
    parity_xent_grad(x, synth.labels(M, N), g, "f32", "signed dloss")


@pytest.mark.parametrize("dtype", DTYPES)
def test_xent_grad_split_rows_are_deterministic(dtype):
    M, N = 300, 131072 if dtype == "f32" else 262144
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    assert rr.rr_plan_query(rr.RR_OP_XENT_GRAD, M, N, code)["path"] == 1
    x = to_dev(synth.normal(M, N, sigma=2.0, dtype=dtype), dtype)
    lab = torch.from_numpy(synth.labels(M, N)).to(DEV)
    g = torch.from_numpy(_dloss(M)).to(DEV)
    ws = rr.workspace(rr.RR_OP_XENT_GRAD, M, N, code, DEV)
    outs = []
    for i in range(REPEATS):
        say("xent grad split-row repeat", i, dtype)
        outs.append(rr.rr_cross_entropy_fwd_bwd(x, lab, g, ws=ws))
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
    for o in outs[1:]:
        assert all(torch.equal(a, b) for a, b in zip(outs[0], o))
    assert rr.rr_workspace_check(ws) == rr.RR_OK
    # gradient rows sum to zero up to the rounding of their entries
    s = outs[0][2].double().sum(dim=1).abs().max()
    assert float(s) < (1e-3 if dtype == "f32" else 0.1)


def test_xent_grad_golden_cases():
    import json
    import os
    say("xent grad golden")
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_cases.json")
    for c in json.load(open(path))["cases"]:
        if c["op"] != "xent_grad":
            continue
        x = np.array([[float.fromhex(v) for v in r] for r in c["x"]], dtype=np.float32)
        lab = np.array(c["labels"], np.int32)
        g = np.array([float.fromhex(v) for v in c["dloss"]], dtype=np.float32)
        loss, lse, dx = run_xent_grad(x, lab, g, "f32")
        check_f32(loss, np.array([float(v) for v in c["loss"]]), c["name"] + " loss")
        check_f32(lse, np.array([float(v) for v in c["lse"]]), c["name"] + " lse")
        ref = np.array([[float(v) for v in r] for r in c["dx"]])
        check_grad(dx, ref, xent_grad_scale(x, lab, g), "f32", c["name"] + " dx")


# ------------------------------------------------------------- softmax backward

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", SHAPES)
def test_softmax_bwd(M, N, dtype):
    say("softmax bwd", dtype, M, N)
    y, dy = softmax_bwd_inputs(M, N, dtype)
    parity_softmax_bwd(y, dy, dtype, f"softmax bwd {dtype} {M}x{N}")


SMBWD_FORCED = [("stream", 32, 512, 2, 300, 20000), ("stream", 32, 512, 16, 97, 70000),
                ("stream", 16, 1024, 1, 700, 16000), ("stream", 16, 1024, 16, 9, 262144),
                ("stream", 32, 512, 1, 3, 16384), ("block", 16, 16, 1, 100, 256),
                ("block", 32, 128, 1, 31, 4000), ("block", 64, 512, 1, 5, 32768),
                ("block", 32, 1024, 1, 6, 30000), ("block", 8, 64, 1, 70, 300),
                ("stream", 32, 512, 32, 40, 500000), ("stream", 32, 512, 64, 3, 1 << 20)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind,P,R,G,M,N", SMBWD_FORCED)
def test_softmax_bwd_forced_plans(kind, P, R, G, M, N, dtype):
    with forced(P, R, G, kind=kind):
        try:
            rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, M, N, rr.RR_F32 if dtype == "f32" else rr.RR_BF16)
        except rr.RRError:
            pytest.skip("not compiled for this dtype (register budget)")
        say("softmax bwd forced", kind, P, R, G, dtype, M, N)
        y, dy = softmax_bwd_inputs(M, N, dtype)
        parity_softmax_bwd(y, dy, dtype, f"softmax bwd {kind} {P},{R},{G}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", [(2, (1 << 20) + 8), (1, 3_000_000), (3, 1_500_016)])
def test_softmax_bwd_long_rows(M, N, dtype):
    """Rows past the on-chip plans: the two-read kernel (y and dy summed over a first
    read, dx written from a second), 16 to 64 workgroups per row, ragged last tiles."""
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, M, N, code)["path"] == 4
    say("softmax bwd long", dtype, M, N)
    y, dy = softmax_bwd_inputs(M, N, dtype)
    parity_softmax_bwd(y, dy, dtype, f"softmax bwd long {dtype} {M}x{N}")
    for inplace in ("y", "dy"):  # dx over y or dy: each tile is read before it is written
        say("softmax bwd long in place", inplace, dtype, M, N)
        parity_softmax_bwd(y, dy, dtype, f"softmax bwd long in place {inplace}", inplace=inplace)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", [(7, 1000), (33, 40000), (5, 16 * 16384 + 5), (70, 9)])
def test_softmax_bwd_long_row_kernel_forced_at_short_rows(M, N, dtype):
    """The two-read kernel forced on short rows: tiles that do not fill a row group
    (members with no tile at all), ragged tails, rows of fewer than 16 bytes."""
    with forced(kind="long"):
        say("softmax bwd long forced", dtype, M, N)
        y, dy = softmax_bwd_inputs(M, N, dtype)
        parity_softmax_bwd(y, dy, dtype, f"softmax bwd long forced {dtype} {M}x{N}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("inplace", ["y", "dy"])
def test_softmax_bwd_in_place(inplace, dtype):
    for M, N in ((64, 1024), (8, 131072)):
        say("softmax bwd in place", inplace, dtype, M, N)
        y, dy = softmax_bwd_inputs(M, N, dtype)
        parity_softmax_bwd(y, dy, dtype, f"softmax bwd in place {inplace}", inplace=inplace)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("N", [64, 1000, 4096, 40000, 131072, 300001])
def test_softmax_bwd_unaligned(N, dtype):
    M = 6
    y_np, dy_np = softmax_bwd_inputs(M, N, dtype)
    pad = lambda a: to_dev(np.concatenate([np.zeros(1, a.dtype), a.ravel()]), dtype)[1:].view(M, N)
    y, dy = pad(y_np), pad(dy_np)
    dx = torch.empty(M * N + 1, dtype=y.dtype, device=DEV)[1:].view(M, N)
    assert y.data_ptr() % 16 != 0
    say("softmax bwd unaligned", dtype, N)
    rr.rr_softmax_bwd(y, dy, dx=dx)
    torch.cuda.synchronize()
    check_grad(from_dev(dx), oracle.softmax_backward(y_np, dy_np),
               softmax_bwd_scale(y_np, dy_np, dtype), dtype, "unaligned softmax bwd")


@pytest.mark.parametrize("dtype", DTYPES)
def test_softmax_bwd_special_rows(dtype):
    say("softmax bwd special rows", dtype)
    # one-hot outputs: no gradient at all; uniform outputs: (dy - mean dy) / N
    N = 4096
    y = np.zeros((3, N), dtype=np.float32)
    y[np.arange(3), [0, 17, N - 1]] = 1.0
    yb = y if dtype == "f32" else synth.f32_to_bf16(y)
    dy = synth.normal(3, N, dtype=dtype, stream=synth.STREAM_DY)
    parity_softmax_bwd(yb, dy, dtype, "one-hot y")
    u = np.full((3, N), 1.0 / N, dtype=np.float32)
    parity_softmax_bwd(u if dtype == "f32" else synth.f32_to_bf16(u), dy, dtype, "uniform y")
    # N = 1: y = 1, dx = 0
    y1 = np.ones((40, 1), dtype=np.float32)
    parity_softmax_bwd(y1 if dtype == "f32" else synth.f32_to_bf16(y1),
                       synth.normal(40, 1, dtype=dtype, stream=synth.STREAM_DY), dtype, "N = 1")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("N", [200, 13])
def test_softmax_bwd_rows_do_not_see_the_next_rows_values(N, dtype):
    """Block kernels whose lane groups hold less than a wave share one buffer across
    the rows of a block, so the registers past a row's end hold the next row's
    values.  An Inf or NaN in the next row's dy must not reach this row's dot product
    (0 * Inf): every row without one is finite and matches the oracle."""
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    M = 64
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, M, N, code)["lanes_per_row"] < 64
    y, dy = softmax_bwd_inputs(M, N, dtype)
    bad = np.arange(1, M, 4)  # the first element of every fourth row
    inf = np.float32(np.inf) if dtype == "f32" else np.uint16(0x7F80)
    nan = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
    dy = dy.copy()
    dy[bad[0::2], 0] = inf
    dy[bad[1::2], 0] = nan
    say("softmax bwd next-row Inf/NaN", dtype, M, N)
    dx = from_dev(rr.rr_softmax_bwd(to_dev(y, dtype), to_dev(dy, dtype)))
    torch.cuda.synchronize()
    good = np.setdiff1d(np.arange(M), bad)
    ref = oracle.softmax_backward(y[good], dy[good])
    got = dx[good]
    got64 = got.astype(np.float64) if dtype == "f32" else \
        (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.isfinite(got64).all(), "a row picked up its neighbour's Inf or NaN"
    check_grad(got, ref, softmax_bwd_scale(y[good], dy[good], dtype), dtype,
               f"softmax bwd rows next to Inf/NaN {dtype} {M}x{N}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_softmax_bwd_split_rows_are_deterministic(dtype):
    M, N = 200, 262144
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, M, N, code)["path"] == 1
    y_np, dy_np = softmax_bwd_inputs(M, N, dtype)
    y, dy = to_dev(y_np, dtype), to_dev(dy_np, dtype)
    ws = rr.workspace(rr.RR_OP_SOFTMAX_BWD, M, N, code, DEV)
    outs = []
    for i in range(REPEATS):
        say("softmax bwd split-row repeat", i, dtype)
        outs.append(rr.rr_softmax_bwd(y, dy, ws=ws))
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    assert rr.rr_workspace_check(ws) == rr.RR_OK
    rows = np.arange(0, M, 37)
    check_grad(from_dev(outs[0][torch.from_numpy(rows).to(DEV)]),
               oracle.softmax_backward(y_np[rows], dy_np[rows]),
               softmax_bwd_scale(y_np[rows], dy_np[rows], dtype), dtype, "split rows sampled")


# ------------------------------------------------------------- RMSNorm backward

RMS_SHAPES = SHAPES + [(1000, 256), (3000, 4096), (4100, 64)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", RMS_SHAPES)
def test_rmsnorm_bwd(M, N, dtype):
    say("rmsnorm bwd", dtype, M, N)
    x, w, dy, r = rmsnorm_bwd_inputs(M, N, dtype)
    parity_rmsnorm_bwd(x, w, dy, r, dtype, f"rmsnorm bwd {dtype} {M}x{N}")


RMS_FORCED = [(8, 16, 1, 300, 100), (8, 1024, 1, 40, 8000), (16, 64, 1, 777, 1000),
              (32, 128, 1, 65, 4000), (16, 512, 2, 300, 9000), (16, 512, 16, 5, 100000),
              (32, 512, 2, 600, 20000), (32, 512, 8, 50, 131072), (32, 512, 16, 3, 200000),
              # 8 and 16 workgroups per row with many rows per row group, ragged shares
              (16, 512, 8, 300, 60000), (16, 512, 16, 100, 131072), (16, 512, 16, 77, 70001)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("P,R,G,M,N", RMS_FORCED)
def test_rmsnorm_bwd_forced_plans(P, R, G, M, N, dtype):
    with forced(P, R, G):
        say("rmsnorm bwd forced", P, R, G, dtype, M, N)
        x, w, dy, r = rmsnorm_bwd_inputs(M, N, dtype)
        parity_rmsnorm_bwd(x, w, dy, r, dtype, f"rmsnorm bwd forced {P},{R},{G}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("inplace", ["x", "dy"])
def test_rmsnorm_bwd_in_place(inplace, dtype):
    for M, N in ((64, 1024), (8, 131072)):
        say("rmsnorm bwd in place", inplace, dtype, M, N)
        x, w, dy, r = rmsnorm_bwd_inputs(M, N, dtype)
        parity_rmsnorm_bwd(x, w, dy, r, dtype, f"rmsnorm bwd in place {inplace}", inplace=inplace)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("N", [64, 1000, 4096, 40000, 131072, 200001, 262144])
def test_rmsnorm_bwd_unaligned(N, dtype):
    M = 6
    x_np, w_np, dy_np, r_np = rmsnorm_bwd_inputs(M, N, dtype)
    pad = lambda a, shape: to_dev(np.concatenate([np.zeros(1, a.dtype), a.ravel()]), dtype)[1:].view(*shape)
    x, dy, w = pad(x_np, (M, N)), pad(dy_np, (M, N)), pad(w_np, (N,))
    dx = torch.empty(M * N + 1, dtype=x.dtype, device=DEV)[1:].view(M, N)
    assert x.data_ptr() % 16 != 0
    say("rmsnorm bwd unaligned", dtype, N)
    dx, dw = rr.rr_rmsnorm_bwd(x, w, dy, torch.from_numpy(r_np).to(DEV), dx=dx)
    torch.cuda.synchronize()
    ref_dx, ref_dw = oracle.rmsnorm_backward(x_np, w_np, dy_np, r_np)
    sdx, sdw = rmsnorm_bwd_scales(x_np, w_np, dy_np, r_np, dtype)
    check_grad(from_dev(dx), ref_dx, sdx, dtype, "unaligned dx")
    check_grad(dw.cpu().numpy(), ref_dw, sdw, "f32", "unaligned dw")


@pytest.mark.parametrize("op", ["xent_grad", "softmax_bwd", "rmsnorm_bwd"])
def test_split_backward_drains_when_the_grid_does_not_fit(op):
    """Row groups forced far beyond what fits at once (row groups are consecutive
    block ids, see the forward test of the same name)."""
    M, N = 200, 262144 if op != "rmsnorm_bwd" else 65536
    say("oversubscribed", op, M, N)
    with forced(groups=M):
        if op == "xent_grad":
            x = synth.normal(M, N, sigma=2.0, dtype="f32")
            parity_xent_grad(x, synth.labels(M, N), _dloss(M), "f32", "oversubscribed xent grad")
        elif op == "softmax_bwd":
            y, dy = softmax_bwd_inputs(M, N, "f32")
            parity_softmax_bwd(y, dy, "f32", "oversubscribed softmax bwd")
        else:
            with forced(16, 512, 8, groups=M):
                parity_rmsnorm_bwd(*rmsnorm_bwd_inputs(M, N, "f32"), "f32",
                                   "oversubscribed rmsnorm bwd")


def test_rmsnorm_bwd_no_rows_gives_zero_dw():
    say("rmsnorm bwd M = 0")
    dw = torch.full((777,), 5.0, device=DEV)
    x = torch.empty((0, 777), device=DEV)
    rr.rr_rmsnorm_bwd(x, torch.ones(777, device=DEV), x, torch.empty(0, device=DEV),
                      dx=x, dw=dw)
    torch.cuda.synchronize()
    assert int(dw.count_nonzero()) == 0


@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_bwd_is_deterministic(dtype):
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    for M, N in ((5000, 4096), (300, 262144)):
        x_np, w_np, dy_np, r_np = rmsnorm_bwd_inputs(M, N, dtype)
        x, w, dy = to_dev(x_np, dtype), to_dev(w_np, dtype), to_dev(dy_np, dtype)
        r = torch.from_numpy(r_np).to(DEV)
        ws = rr.workspace(rr.RR_OP_RMSNORM_BWD, M, N, code, DEV)
        outs = []
        for i in range(REPEATS):
            say("rmsnorm bwd repeat", i, dtype, M, N)
            outs.append(rr.rr_rmsnorm_bwd(x, w, dy, r, ws=ws))
            torch.cuda.synchronize()
        for o in outs[1:]:
            assert torch.equal(outs[0][0], o[0]) and torch.equal(outs[0][1], o[1])
        p = rr.rr_plan_query(rr.RR_OP_RMSNORM_BWD, M, N, code)
        if p["groups_per_row"] > 1:
            assert rr.rr_workspace_check(ws) == rr.RR_OK
        # dw against the oracle on every column, dx on sampled rows
        rows = np.arange(0, M, max(1, M // 16))
        ref_dx, _ = oracle.rmsnorm_backward(x_np[rows], w_np, dy_np[rows], r_np[rows])
        _, ref_dw = oracle.rmsnorm_backward(x_np, w_np, dy_np, r_np)
        sdx, _ = rmsnorm_bwd_scales(x_np[rows], w_np, dy_np[rows], r_np[rows], dtype)
        _, sdw = rmsnorm_bwd_scales(x_np, w_np, dy_np, r_np, dtype)
        check_grad(from_dev(outs[0][0][torch.from_numpy(rows).to(DEV)]), ref_dx, sdx, dtype, "dx")
        check_grad(outs[0][1].cpu().numpy(), ref_dw, sdw, "f32", "dw")


def test_rmsnorm_bwd_golden_cases():
    import json
    import os
    say("rmsnorm bwd golden")
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_cases.json")
    for c in json.load(open(path))["cases"]:
        if c["op"] != "rmsnorm_bwd":
            continue
        x = np.array([[float.fromhex(v) for v in r] for r in c["x"]], dtype=np.float32)
        w = np.array([float.fromhex(v) for v in c["w"]], dtype=np.float32)
        dy = np.array([[float.fromhex(v) for v in r] for r in c["dy"]], dtype=np.float32)
        r = np.array([float.fromhex(v) for v in c["rstd"]], dtype=np.float32)
        dx, dw = rr.rr_rmsnorm_bwd(to_dev(x, "f32"), to_dev(w, "f32"), to_dev(dy, "f32"),
                                   torch.from_numpy(r).to(DEV))
        torch.cuda.synchronize()
        sdx, sdw = rmsnorm_bwd_scales(x, w, dy, r, "f32")
        check_grad(dx.cpu().numpy(), np.array([[float(v) for v in q] for q in c["dx"]]), sdx,
                   "f32", c["name"] + " dx")
        check_grad(dw.cpu().numpy(), np.array([float(v) for v in c["dw"]]), sdw, "f32",
                   c["name"] + " dw")
