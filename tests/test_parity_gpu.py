"""GPU parity: the HIP kernels (through the C ABI) against the double-precision
oracle, element by element, on seeded inputs.

Tolerances (tests/_verify.py): fp32 outputs within relative 1e-5, bf16 outputs
within one bf16 ulp of the exact value.  Sizes are small enough for the oracle to
finish in seconds but span several tiles and ragged tails; every path (one lane
group per row, one workgroup per row, split rows, the per-element path for
unaligned rows) is run, the split-row path also forced at small N with many rows.
"""
import json
import os

import numpy as np
import pytest
import torch

import memory_bound_row_softmax_amd as rr
import oracle
import synth
from _gpu import (DEV, check_out, forced, from_dev, parity_rmsnorm, parity_softmax,
                  parity_xent, run_softmax, say, to_dev, xent_grad_scale)
from _verify import check_f32, check_grad

pytestmark = pytest.mark.gpu

# launches of a determinism test, each compared with the first bit for bit
REPEATS = 20

DTYPES = ("f32", "bf16")
# (M, N): every plan bucket, ragged tails, a few rows past a block boundary
SHAPES = [(256, 1024), (64, 1), (64, 3), (70, 255), (64, 256), (33, 257), (37, 1000), (16, 2048),
          (16, 4095), (16, 4096), (9, 4097), (8, 16384), (5, 20000), (4, 65536), (3, 65537),
          (3, 131072), (2, 200000), (2, 262144)]


def _x(M, N, dtype, sigma=1.0, seed=synth.SEED):
    return synth.normal(M, N, sigma=sigma, dtype=dtype, seed=seed)


def _w(N, dtype):
    return synth.uniform(1, N, lo=0.5, hi=1.5, dtype=dtype).reshape(N)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", SHAPES)
def test_softmax(M, N, dtype):
    say("softmax", dtype, M, N)
    parity_softmax(_x(M, N, dtype, sigma=3.0), dtype, f"softmax {dtype} {M}x{N}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", SHAPES)
def test_rmsnorm(M, N, dtype):
    say("rmsnorm", dtype, M, N)
    parity_rmsnorm(_x(M, N, dtype), _w(N, dtype), 1e-6, dtype, f"rmsnorm {dtype} {M}x{N}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", SHAPES + [(40, 50000)])
def test_cross_entropy(M, N, dtype):
    say("xent", dtype, M, N)
    x = _x(M, N, dtype, sigma=2.0)
    lab = synth.labels(M, N)
    parity_xent(x, lab, dtype, f"xent {dtype} {M}x{N}")


# ------------------------------------------------------------- forced paths

FORCED_ROW = [  # (kind, P, R, G, M, N): split rows at small N, empty / partial member
    # slices, many rows per persistent workgroup, block kernels off their default sizes
    ("stream", 64, 256, 2, 300, 20000), ("stream", 64, 256, 4, 300, 3000),
    ("stream", 32, 512, 16, 97, 70000), ("stream", 64, 512, 2, 50, 65536),
    ("stream", 32, 1024, 2, 40, 65536), ("stream", 64, 512, 16, 9, 500000),
    ("stream", 16, 1024, 1, 700, 16000), ("stream", 64, 256, 1, 1000, 5000),
    ("stream", 32, 512, 1, 3, 16384), ("stream", 16, 1024, 8, 200, 100000),
    ("block", 16, 16, 1, 100, 256), ("block", 32, 128, 1, 31, 4000),
    ("block", 16, 1024, 1, 5, 16384), ("block", 8, 512, 1, 77, 3000),
    ("block", 64, 1024, 1, 6, 65536),
    # deferred exchange (8 or more workgroups per row): many rows per row group, so
    # the four slot sets are reused many times over
    ("stream", 64, 512, 8, 333, 200000), ("stream", 16, 1024, 16, 150, 250000),
    ("stream", 16, 1024, 8, 1000, 70000),
    # 128 workgroups per row: most members hold nothing of a short row; 10 rows per
    # row group
    ("stream", 64, 512, 128, 20, 100000)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind,P,R,G,M,N", FORCED_ROW)
def test_forced_row_plans(kind, P, R, G, M, N, dtype):
    ran = 0
    for op in ("softmax", "rmsnorm"):
        code = rr.RR_OP_SOFTMAX if op == "softmax" else rr.RR_OP_RMSNORM
        with forced(P, R, G, kind=kind):
            try:
                rr.rr_plan_query(code, M, N, rr.RR_F32 if dtype == "f32" else rr.RR_BF16)
            except rr.RRError:
                continue  # not compiled for this op (register budget)
            say(op, "forced", kind, P, R, G, dtype, M, N)
            ran += 1
            if op == "softmax":
                parity_softmax(_x(M, N, dtype, sigma=2.0), dtype, f"softmax {kind} {P},{R},{G}")
            else:
                parity_rmsnorm(_x(M, N, dtype), _w(N, dtype), 1e-6, dtype,
                               f"rmsnorm {kind} {P},{R},{G}")
    assert ran > 0


EXACT_GROUPS = [(3, 70000), (5, 151936), (6, 180000)]


@pytest.mark.parametrize("G,N", EXACT_GROUPS)
def test_bf16_softmax_takes_exactly_the_workgroups_a_row_needs(G, N):
    """bf16 rows on 64 values x 512 lanes are split over ceil(N / 32768) workgroups,
    also when that is 3, 5 or 6, with 40 rows so that each row group has several."""
    M = 40
    p = rr.rr_plan_query(rr.RR_OP_SOFTMAX, 16384, N, rr.RR_BF16)
    assert (p["path"], p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]) == (1, 64, 512, G)
    say("softmax exact groups", G, M, N)
    with forced(groups=2):  # two row groups: 20 rows each, every slot set reused
        parity_softmax(_x(M, N, "bf16", sigma=2.0), "bf16", f"softmax bf16 G={G} {M}x{N}")
    parity_softmax(_x(M, N, "bf16", sigma=2.0), "bf16", f"softmax bf16 G={G} {M}x{N}")


@pytest.mark.parametrize("G,N", EXACT_GROUPS)
def test_fp32_softmax_exact_groups(G, N):
    """fp32 rows on 64 values x 512 lanes split over 3, 5 or 6 workgroups (the planner
    picks 5 and 6; 3 is forced), one contiguous part per workgroup, the last shorter."""
    M = 40
    if G != 3:
        p = rr.rr_plan_query(rr.RR_OP_SOFTMAX, 16384, N, rr.RR_F32)
        assert (p["path"], p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]) == (1, 64, 512, G)
    say("softmax fp32 exact groups", G, M, N)
    with forced(64, 512, G, kind="stream", groups=2):
        parity_softmax(_x(M, N, "f32", sigma=2.0), "f32", f"softmax f32 G={G} {M}x{N}")
    with forced(64, 512, G, kind="stream"):
        parity_softmax(_x(M, N, "f32", sigma=2.0), "f32", f"softmax f32 G={G} {M}x{N}")


PACKED = [  # (G, M, N): packed bf16 RMSNorm (128 values per lane on 512 lanes)
    (1, 300, 65536), (1, 700, 20000), (1, 3, 8), (2, 100, 131072), (2, 61, 65544),
    (4, 90, 200000), (8, 40, 524288), (16, 7, 1000000), (16, 5, 300000), (16, 33, 1 << 20),
    (64, 5, 1 << 22), (64, 9, 3_000_000), (128, 3, 1 << 23), (128, 4, 6_000_000),
    (256, 2, 1 << 24), (256, 3, 15_000_000)]


@pytest.mark.parametrize("G,M,N", PACKED)
def test_packed_bf16_rmsnorm(G, M, N):
    """bf16 rows kept as raw chunks: one workgroup up to 65536 elements, then split;
    ragged rows, members with an empty part (300000 on 16), many rows per group."""
    with forced(128, 512, G, kind="stream"):
        p = rr.rr_plan_query(rr.RR_OP_RMSNORM, M, N, rr.RR_BF16)
        assert p["vals_per_lane"] == 128 and p["groups_per_row"] == G
        say("rmsnorm packed", G, M, N)
        parity_rmsnorm(_x(M, N, "bf16", sigma=2.0), _w(N, "bf16"), 1e-6, "bf16",
                       f"rmsnorm packed {G} {M}x{N}")
        # only RMSNorm, only bf16, only on the 128-bit path
        for args in ((rr.RR_OP_RMSNORM, M, N, rr.RR_F32), (rr.RR_OP_RMSNORM, M, N, rr.RR_BF16, False),
                     (rr.RR_OP_SOFTMAX, M, N, rr.RR_BF16), (rr.RR_OP_XENT_GRAD, M, N, rr.RR_BF16)):
            with pytest.raises(rr.RRError):
                rr.rr_plan_query(*args)


@pytest.mark.parametrize("dtype,P,G,N", [("f32", 64, 16, 524288), ("f32", 64, 32, 1_000_000),
                                         ("f32", 64, 64, 2_097_152), ("bf16", 128, 16, 1_000_000),
                                         ("bf16", 128, 32, 2_000_000)])
def test_rmsnorm_deferred_many_rows_per_group(dtype, P, G, N):
    """RMSNorm rows on 512 lanes defer the exchange from 16 workgroups (64 fp32 values,
    or 128 packed bf16 ones): two row groups give each of them many rows, so every
    exchange slot set is reused; ragged rows leave the last members' parts short."""
    M = 11
    with forced(P, 512, G, kind="stream", groups=2):
        p = rr.rr_plan_query(rr.RR_OP_RMSNORM, M, N, rr.RR_F32 if dtype == "f32" else rr.RR_BF16)
        assert (p["vals_per_lane"], p["groups_per_row"]) == (P, G)
        say("rmsnorm deferred", dtype, P, G, M, N)
        parity_rmsnorm(_x(M, N, dtype, sigma=2.0), _w(N, dtype), 1e-6, dtype,
                       f"rmsnorm deferred {dtype} {G} {M}x{N}")


@pytest.mark.parametrize("M,N", [(300, 262144), (77, 200000), (40, 131080), (9, 65536)])
def test_packed_bf16_rmsnorm_on_256_lanes(M, N):
    """Packed bf16 RMSNorm on 8 workgroups of 256 lanes (the plan from 131073 to 262144
    elements): full, ragged and short rows (members with an empty part)."""
    if N > 131072:
        p = rr.rr_plan_query(rr.RR_OP_RMSNORM, 16384, N, rr.RR_BF16)
        assert (p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]) == (128, 256, 8), p
    with forced(128, 256, 8, kind="stream"):
        say("rmsnorm packed 256x8", M, N)
        parity_rmsnorm(_x(M, N, "bf16", sigma=2.0), _w(N, "bf16"), 1e-6, "bf16",
                       f"rmsnorm packed 256x8 {M}x{N}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("P,R", [(16, 16), (16, 1024), (32, 64), (32, 512)])
def test_forced_xent_plans(P, R, dtype):
    M, N = 45, 7777
    with forced(P, R):
        say("xent forced", P, R, dtype)
        parity_xent(_x(M, N, dtype, sigma=2.0), synth.labels(M, N), dtype, f"xent forced {P},{R}")


# ------------------------------------------------------------- layouts

@pytest.mark.parametrize("N", [16385, 20001, 50257, 65537, 81919, 81921])
def test_unaligned_bf16_split_rows_wide_lanes(N):
    """Unaligned bf16 softmax and RMSNorm rows of 16385 to 81920 elements: 32 values on
    512 lanes over 2 to 8 workgroups (16 on 1024 past that), with a base one element
    past a 16-byte boundary and 40 rows, so row groups take several rows.  The
    cross-entropy gradient takes them past 32768 elements."""
    M = 40
    wide = N <= 81920
    for code in (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM, rr.RR_OP_XENT_GRAD):
        p = rr.rr_plan_query(code, M, N, rr.RR_BF16, False)
        if code == rr.RR_OP_XENT_GRAD and N <= 32768:
            continue  # the table's block kernels
        assert (p["vals_per_lane"], p["lanes_per_row"]) == ((32, 512) if wide else (16, 1024))
        assert 2 <= p["groups_per_row"] <= (8 if wide else 16)
    x_np = _x(M, N, "bf16", sigma=2.0)
    w_np = _w(N, "bf16")
    xs = to_dev(np.concatenate([np.zeros(1, x_np.dtype), x_np.ravel()]), "bf16")[1:].view(M, N)
    ys = torch.empty(M * N + 1, dtype=xs.dtype, device=DEV)[1:].view(M, N)
    wt = torch.empty(N + 1, dtype=xs.dtype, device=DEV)[1:]
    wt.copy_(to_dev(w_np, "bf16"))
    say("unaligned wide softmax", N)
    rr.rr_softmax_fwd(xs, ys, ws=rr.workspace(rr.RR_OP_SOFTMAX, M, N, rr.RR_BF16, DEV))
    torch.cuda.synchronize()
    check_out(from_dev(ys), oracle.softmax(x_np), "bf16", f"unaligned wide softmax {N}")
    say("unaligned wide rmsnorm", N)
    rr.rr_rmsnorm_fwd(xs, wt, 1e-6, y=ys, ws=rr.workspace(rr.RR_OP_RMSNORM, M, N, rr.RR_BF16, DEV))
    torch.cuda.synchronize()
    check_out(from_dev(ys), oracle.rmsnorm(x_np, w_np, 1e-6), "bf16", f"unaligned wide rmsnorm {N}")
    say("unaligned wide xent grad", N)
    lab = synth.labels(M, N)
    g = synth.uniform(1, M, lo=0.5, hi=1.5, stream=synth.STREAM_DLOSS)[0]
    loss, lse, dx = rr.rr_cross_entropy_fwd_bwd(xs, torch.from_numpy(lab).to(DEV),
                                                torch.from_numpy(g).to(DEV), dlogits=ys)
    torch.cuda.synchronize()
    ref_loss, ref_lse, ref_dx = oracle.cross_entropy_grad(x_np, lab, g)
    check_f32(loss.cpu().numpy(), ref_loss, f"unaligned wide xent grad loss {N}")
    check_f32(lse.cpu().numpy(), ref_lse, f"unaligned wide xent grad lse {N}")
    check_grad(from_dev(dx), ref_dx, xent_grad_scale(x_np, lab, g), "bf16",
               f"unaligned wide xent grad dx {N}")


UNALIGNED_ROWS = [  # (kind, P, R, G, N): aligned tensors whose row length is not a
    # multiple of 16 bytes, so the rows start at every offset modulo 16 bytes
    ("block", 16, 512, 1, 5001), ("block", 32, 256, 1, 8191), ("stream", 16, 1024, 1, 16001),
    ("stream", 16, 1024, 2, 30001), ("stream", 32, 512, 4, 50257),
    ("stream", 16, 1024, 8, 120001), ("stream", 16, 1024, 16, 250001),
    ("stream", 16, 1024, 1, 16383), ("stream", 16, 1024, 1, 16381)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind,P,R,G,N", UNALIGNED_ROWS)
def test_rows_at_every_offset(kind, P, R, G, N, dtype):
    """Softmax and the cross-entropy gradient on 37 rows that start at every offset
    modulo 16 bytes, on forced per-element plans, element by element against the
    oracle."""
    M = 37
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    with forced(P, R, G, kind=kind):
        try:
            rr.rr_plan_query(rr.RR_OP_SOFTMAX, M, N, code, False)
        except rr.RRError:
            pytest.skip("not compiled for this dtype")
        say("rows at every offset", kind, P, R, G, dtype, M, N)
        x_np = _x(M, N, dtype, sigma=2.0)
        parity_softmax(x_np, dtype, f"offset rows softmax {kind} {P},{R},{G} {N}")
        lab = synth.labels(M, N)
        g = synth.uniform(1, M, lo=0.5, hi=1.5, stream=synth.STREAM_DLOSS)[0]
        loss, lse, dx = rr.rr_cross_entropy_fwd_bwd(to_dev(x_np, dtype), torch.from_numpy(lab).to(DEV),
                                                    torch.from_numpy(g).to(DEV))
        torch.cuda.synchronize()
        ref_loss, ref_lse, ref_dx = oracle.cross_entropy_grad(x_np, lab, g)
        check_f32(loss.cpu().numpy(), ref_loss, f"offset rows xent grad loss {N}")
        check_f32(lse.cpu().numpy(), ref_lse, f"offset rows xent grad lse {N}")
        check_grad(from_dev(dx), ref_dx, xent_grad_scale(x_np, lab, g), dtype,
                   f"offset rows xent grad dx {kind} {P},{R},{G} {N}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("N", [64, 1000, 4096, 40000, 131072])
def test_unaligned_rows_take_the_element_path(N, dtype):
    M = 6
    x_np = _x(M, N, dtype, sigma=2.0)
    w_np = _w(N, dtype)
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    # the tensors start one element past a 16-byte boundary
    xs = to_dev(np.concatenate([np.zeros(1, x_np.dtype), x_np.ravel()]), dtype)[1:].view(M, N)
    ys = torch.empty(M * N + 1, dtype=xs.dtype, device=DEV)[1:].view(M, N)
    wt = torch.empty(N + 1, dtype=xs.dtype, device=DEV)[1:]
    wt.copy_(to_dev(w_np, dtype))
    assert xs.data_ptr() % 16 != 0 and wt.data_ptr() % 16 != 0
    say("unaligned softmax", dtype, N)
    rr.rr_softmax_fwd(xs, ys, ws=rr.workspace(rr.RR_OP_SOFTMAX, M, N, code, DEV))
    torch.cuda.synchronize()
    check_out(from_dev(ys), oracle.softmax(x_np), dtype, "unaligned softmax")
    say("unaligned rmsnorm", dtype, N)
    rr.rr_rmsnorm_fwd(xs, wt, 1e-6, y=ys, ws=rr.workspace(rr.RR_OP_RMSNORM, M, N, code, DEV))
    torch.cuda.synchronize()
    check_out(from_dev(ys), oracle.rmsnorm(x_np, w_np, 1e-6), dtype, "unaligned rmsnorm")
    say("unaligned xent", dtype, N)
    lab = synth.labels(M, N)
    loss, lse = rr.rr_cross_entropy_fwd(xs, torch.from_numpy(lab).to(DEV))
    ref_loss, ref_lse = oracle.cross_entropy(x_np, lab)
    check_f32(lse.cpu().numpy(), ref_lse, "unaligned lse")
    check_f32(loss.cpu().numpy(), ref_loss, "unaligned loss")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", [(64, 1024), (8, 131072)])
def test_in_place(M, N, dtype):
    x_np = _x(M, N, dtype, sigma=2.0)
    say("in-place softmax", dtype, M, N)
    got = run_softmax(x_np, dtype, inplace=True)
    check_out(got, oracle.softmax(x_np), dtype, "in-place softmax")
    say("in-place rmsnorm", dtype, M, N)
    w_np = _w(N, dtype)
    x = to_dev(x_np, dtype)
    rr.rr_rmsnorm_fwd(x, to_dev(w_np, dtype), 1e-6, y=x)
    torch.cuda.synchronize()
    check_out(from_dev(x), oracle.rmsnorm(x_np, w_np, 1e-6), dtype, "in-place rmsnorm")


# ------------------------------------------------------------- special values

@pytest.mark.parametrize("dtype", DTYPES)
def test_closed_forms(dtype):
    say("closed forms", dtype)
    # constant rows: softmax = 1/N exactly; CE = ln N; RMSNorm = w * c / sqrt(c^2 + eps)
    for N in (1, 4096, 131072):
        c = np.full((4, N), 2.5, dtype=np.float32)
        x = c if dtype == "f32" else synth.f32_to_bf16(c)
        y = run_softmax(x, dtype)
        y = y if dtype == "f32" else (y.astype(np.uint32) << 16).view(np.float32)
        assert np.all(y == np.float32(1.0 / N)), N
        parity_xent(x, np.zeros(4, np.int32), dtype, "constant xent")
        parity_rmsnorm(x, _w(N, dtype), 1e-6, dtype, "constant rmsnorm")
    # N = 1: softmax 1, cross-entropy 0
    x = _x(50, 1, dtype, sigma=5.0)
    y = run_softmax(x, dtype)
    y = y if dtype == "f32" else (y.astype(np.uint32) << 16).view(np.float32)
    assert np.all(y == 1.0)
    lab = np.zeros(50, np.int32)
    x_dev = to_dev(x, dtype)
    loss, lse = rr.rr_cross_entropy_fwd(x_dev, torch.from_numpy(lab).to(DEV))
    torch.cuda.synchronize()
    assert np.all(loss.cpu().numpy() == 0.0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_spiky_and_large_rows(dtype):
    say("spiky / large rows", dtype)
    x = _x(40, 8192, dtype)
    synth.spikes_(x, p=0.01, value=20.0, dtype=dtype)
    parity_softmax(x, dtype, "spiky softmax")
    parity_xent(x, synth.labels(40, 8192), dtype, "spiky xent")
    big = (_x(8, 3000, "f32") * 30 + 1000.0).astype(np.float32)
    big = big if dtype == "f32" else synth.f32_to_bf16(big)
    parity_softmax(big, dtype, "large-value softmax")
    parity_xent(big, synth.labels(8, 3000), dtype, "large-value xent")


@pytest.mark.parametrize("dtype", DTYPES)
def test_invalid_labels_give_nan(dtype):
    say("invalid labels", dtype)
    M, N = 8, 5000
    x = _x(M, N, dtype, sigma=2.0)
    lab = np.array([0, -1, N, N - 1, 1 << 30, 7, -(1 << 30), 4999], dtype=np.int32)
    parity_xent(x, lab, dtype, "invalid labels")


def test_nan_input_propagates():
    say("nan input")
    x = _x(4, 3000, "f32")
    x[1, 17] = np.nan
    got = run_softmax(x, "f32")
    assert np.all(np.isnan(got[1])) and np.all(np.isfinite(got[[0, 2, 3]]))


def test_golden_cases():
    say("golden cases")
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_cases.json")
    for c in json.load(open(path))["cases"]:
        if c["dtype"] == "f32":
            x = np.array([[float.fromhex(v) for v in r] for r in c["x"]], dtype=np.float32)
            w = np.array([float.fromhex(v) for v in c["w"]], dtype=np.float32) if "w" in c else None
        else:
            x = np.array([[int(v, 16) for v in r] for r in c["x"]], dtype=np.uint16)
            w = np.array([int(v, 16) for v in c["w"]], dtype=np.uint16) if "w" in c else None
        if c["op"] == "softmax":
            ref = np.array([[float(v) for v in r] for r in c["y"]])
            check_out(run_softmax(x, c["dtype"]), ref, c["dtype"], c["name"])
        elif c["op"] == "rmsnorm":
            from _gpu import run_rmsnorm
            ref = np.array([[float(v) for v in r] for r in c["y"]])
            check_out(run_rmsnorm(x, w, c["eps"], c["dtype"]), ref, c["dtype"], c["name"])
        elif c["op"] == "xent":
            from _gpu import run_xent
            loss, lse = run_xent(x, np.array(c["labels"], np.int32), c["dtype"])
            check_f32(lse, np.array([float(v) for v in c["lse"]]), c["name"] + " lse")
            check_f32(loss, np.array([float(v) for v in c["loss"]]), c["name"] + " loss")


# ------------------------------------------------------------- grid path hygiene

@pytest.mark.parametrize("dtype", DTYPES)
def test_split_rows_are_deterministic_and_leave_the_workspace_zero(dtype):
    M, N = 600, 131072 if dtype == "f32" else 262144
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, M, N, code)["path"] == 1
    x = to_dev(_x(M, N, dtype, sigma=2.0), dtype)
    ws = rr.workspace(rr.RR_OP_SOFTMAX, M, N, code, DEV)
    outs = []
    for i in range(REPEATS):
        say("split-row repeat", i, dtype)
        y = rr.rr_softmax_fwd(x, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
        outs.append(y)
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    assert rr.rr_workspace_check(ws) == rr.RR_OK
    # rows sum to 1 (in double) on every row
    s = outs[0].double().sum(dim=1)
    assert float((s - 1).abs().max()) < (1e-4 if dtype == "f32" else 2e-2)


# Split-row calls for the timeout tests: (name, op, dtype, M, N, forced kind).  Each
# takes a plan whose rows are split over several workgroups (or read twice by the
# long-row kernel), with the exchange inside a row's step and deferred.
TIMEOUT_CASES = [
    ("softmax f32 G4", "softmax", "f32", 64, 131072, None),
    ("softmax f32 G8 deferred", "softmax", "f32", 64, 262144, None),
    ("softmax bf16 G4", "softmax", "bf16", 64, 262144, None),
    ("rmsnorm f32 G8", "rmsnorm", "f32", 64, 262144, None),
    ("rmsnorm bf16 packed G4", "rmsnorm", "bf16", 64, 262144, None),
    ("xent_grad f32 G4", "xent_grad", "f32", 64, 131072, None),
    ("softmax_bwd f32 G8 deferred", "softmax_bwd", "f32", 64, 262144, None),
    ("rmsnorm_bwd f32 G4", "rmsnorm_bwd", "f32", 64, 65536, None),
    ("long-row softmax", "softmax", "f32", 48, 70000, "long"),
    ("long-row rmsnorm", "rmsnorm", "bf16", 48, 70000, "long"),
    ("rmsnorm f32 G16 deferred", "rmsnorm", "f32", 64, 524288, None),
    ("rmsnorm bf16 packed G16 deferred", "rmsnorm", "bf16", 64, 1 << 20, None),
    ("long-row softmax_bwd", "softmax_bwd", "f32", 48, 70000, "long"),
    ("long-row xent_grad", "xent_grad", "bf16", 48, 70000, "long"),
]

_OP_CODES = {"softmax": rr.RR_OP_SOFTMAX, "rmsnorm": rr.RR_OP_RMSNORM,
             "xent_grad": rr.RR_OP_XENT_GRAD, "softmax_bwd": rr.RR_OP_SOFTMAX_BWD,
             "rmsnorm_bwd": rr.RR_OP_RMSNORM_BWD}


def _split_call(op, dtype, M, N, kind):
    """Inputs and a launcher for one split-row call; the launcher returns the row
    outputs as float64 arrays ([M, N] matrices and [M] vectors) and dw (or None)."""
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    with forced(kind=kind):
        plan = rr.rr_plan_query(_OP_CODES[op], M, N, code)
        ws = rr.workspace(_OP_CODES[op], M, N, code, DEV)
    assert plan["path"] in (1, 4), plan
    x_np = _x(M, N, dtype, sigma=2.0)
    x = to_dev(x_np, dtype)
    w = to_dev(_w(N, dtype), dtype)
    dy = to_dev(synth.normal(M, N, dtype=dtype, stream=synth.STREAM_DY), dtype)
    lab = torch.from_numpy(synth.labels(M, N)).to(DEV)
    g = torch.full((M,), 0.5, dtype=torch.float32, device=DEV)
    rstd = torch.empty(M, dtype=torch.float32, device=DEV)
    rr.rr_rmsnorm_fwd(x, w, 1e-6, rstd=rstd)
    yfwd = rr.rr_softmax_fwd(x)
    torch.cuda.synchronize()

    def run(spin=None):
        with forced(kind=kind, spin=spin):
            if op == "softmax":
                outs, dw = [rr.rr_softmax_fwd(x, ws=ws)], None
            elif op == "rmsnorm":
                r = torch.empty(M, dtype=torch.float32, device=DEV)
                outs, dw = [rr.rr_rmsnorm_fwd(x, w, 1e-6, rstd=r, ws=ws), r], None
            elif op == "xent_grad":
                loss, lse, dx = rr.rr_cross_entropy_fwd_bwd(x, lab, g, ws=ws)
                outs, dw = [dx, loss, lse], None
            elif op == "softmax_bwd":
                outs, dw = [rr.rr_softmax_bwd(yfwd, dy, ws=ws)], None
            else:
                dx, dw = rr.rr_rmsnorm_bwd(x, w, dy, rstd, ws=ws)
                outs = [dx]
        torch.cuda.synchronize()
        return [o.double().cpu().numpy() for o in outs], dw

    return ws, run


def _exchange_area(ws, op, dtype, M, N):
    """The part of a workspace that must be zero between launches: all of it, except
    for the RMSNorm backward's dw partial rows (scratch every call rewrites), which
    follow the header and the exchange area of its 128-bit plan: 256 bytes, then for
    split rows min(parts, 1024) records of 64 + 64 G bytes, parts = min(row blocks,
    1024 / G), rounded up to 256 bytes."""
    if op != "rmsnorm_bwd":
        return ws
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    p = rr.rr_plan_query(rr.RR_OP_RMSNORM_BWD, M, N, code)
    G = p["groups_per_row"]
    if G == 1:
        return ws[:256]
    parts = min(-(-M // p["rows_per_block"]), 1024 // G)
    exch = 256 + min(parts, 1024) * (64 + 64 * G)
    return ws[:-(-exch // 256) * 256]


@pytest.mark.parametrize("name,op,dtype,M,N,kind", TIMEOUT_CASES)
def test_forced_timeout_gives_nan_rows_and_is_reported(name, op, dtype, M, N, kind):
    """With every split-row wait forced to give up at once (spin limit -1, set from
    the host), the kernel must still finish, write NaN for every value of every split
    row (never a wrong number), report RR_ERR_GRID_TIMEOUT and leave the workspace
    clean; a normal call afterwards gives the same bits as a call before."""
    ws, run = _split_call(op, dtype, M, N, kind)
    say("reference call", name)
    ref, ref_dw = run()
    assert rr.rr_workspace_check(ws) == rr.RR_OK
    say("forced timeout", name)
    outs, dw = run(spin=-1)
    assert rr.rr_workspace_check(ws) == rr.RR_ERR_GRID_TIMEOUT
    # error word cleared by the check, slots by the kernel
    assert int(_exchange_area(ws, op, dtype, M, N).count_nonzero()) == 0
    for o in outs:
        assert np.isnan(o).all(), f"{name}: a timed-out split row holds a non-NaN value"
    if dw is not None:  # dw does not depend on the exchange
        assert torch.equal(dw, ref_dw)
    say("after timeout", name)
    again, _ = run()
    assert rr.rr_workspace_check(ws) == rr.RR_OK
    for a, b in zip(again, ref):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name,op,dtype,M,N,kind", TIMEOUT_CASES[:2] + TIMEOUT_CASES[5:8] + TIMEOUT_CASES[10:])
def test_one_poll_waits_never_give_silent_garbage(name, op, dtype, M, N, kind):
    """With a spin limit of one poll, some waits may give up and others succeed.
    Every row must then be either exactly the normal result or hold NaN, and a row
    with NaN must come with RR_ERR_GRID_TIMEOUT."""
    ws, run = _split_call(op, dtype, M, N, kind)
    say("reference call", name)
    ref, _ = run()
    say("one-poll waits", name)
    outs, _ = run(spin=1)
    st = rr.rr_workspace_check(ws)
    assert st in (rr.RR_OK, rr.RR_ERR_GRID_TIMEOUT)
    assert int(_exchange_area(ws, op, dtype, M, N).count_nonzero()) == 0
    any_nan = False
    for o, r in zip(outs, ref):
        rows_nan = np.isnan(o).reshape(M, -1).any(axis=1)
        any_nan |= bool(rows_nan.any())
        ok = rows_nan | (o == r).reshape(M, -1).all(axis=1)
        assert ok.all(), f"{name}: rows {np.flatnonzero(~ok)[:5]} differ without NaN"
    if any_nan:
        assert st == rr.RR_ERR_GRID_TIMEOUT


OVERSUBSCRIBED = [  # (op, dtype, M, N): row groups forced to M, far more than fit at once
    # A row group is G consecutive block ids, spread over the 8 XCDs (block b on
    # XCD b mod 8), so a forced grid drains when each XCD (32 CUs) holds ceil(G / 8)
    # workgroups at once.
    ("softmax", "f32", 256, 200000),    # 8 workgroups per row, deferred exchange: 2048
    ("softmax", "bf16", 64, 1 << 20),   # 32 per row: 2048
    ("rmsnorm", "bf16", 256, 262144),   # packed, 4 per row: 1024 (one fits per CU)
    ("rmsnorm", "f32", 96, 1 << 19),    # 32 per row: 3072
    ("softmax", "f32", 64, 2_000_000),  # 64 per row: 4096
    ("softmax", "f32", 32, 4_000_000),  # 128 per row: 4096
    ("softmax", "f32", 64, 3_000_000),  # two-pass long rows, 32 per row: 2048 (two per CU)
    ("softmax", "f32", 16, 5_000_000),  # two-pass long rows, 64 per row: 1024 (two per CU)
]


@pytest.mark.parametrize("op,dtype,M,N", OVERSUBSCRIBED)
def test_split_rows_drain_when_the_grid_does_not_fit(op, dtype, M, N):
    """Workgroups that share a row wait for each other, and an ordinary launch does
    not promise that the whole grid runs at once.  A row group is G consecutive
    block ids and each XCD starts its blocks in id order, so a grid several times
    larger than the device holds must still drain, with every row right and the
    workspace left clean, as long as each XCD can hold ceil(G / 8) of them."""
    code = {"softmax": rr.RR_OP_SOFTMAX, "rmsnorm": rr.RR_OP_RMSNORM}[op]
    dt = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    assert rr.rr_plan_query(code, M, N, dt)["groups_per_row"] > 1
    x_np = _x(M, N, dtype, sigma=2.0)
    x = to_dev(x_np, dtype)
    ws = rr.workspace(code, M, N, dt, DEV)
    say("oversubscribed", op, dtype, M, N)
    with forced(groups=M):
        if op == "softmax":
            y = rr.rr_softmax_fwd(x, ws=ws)
            ref = oracle.softmax(x_np)
        else:
            w_np = _w(N, dtype)
            y = rr.rr_rmsnorm_fwd(x, to_dev(w_np, dtype), 1e-6, ws=ws)
            ref = oracle.rmsnorm(x_np, w_np, 1e-6)
        torch.cuda.synchronize()
    assert rr.rr_workspace_check(ws) == rr.RR_OK
    assert int(ws.count_nonzero()) == 0
    check_out(from_dev(y), ref, dtype, f"oversubscribed {op} {dtype} {M}x{N}")


@pytest.mark.parametrize("nbytes", [16, 1024 + 16, 3 * 131072 + 4096 + 32, 1 << 22,
                                    (1 << 32) + 48])
def test_streams(nbytes):
    """The copy, read and fill streams (the bench's ceilings) move exactly `nbytes`,
    including a partial last region and offsets past 32 bits: the copy is exact and
    leaves the bytes after it alone, the read's checksums XOR to the data's, and the
    fill writes the pattern and nothing after it."""
    say("streams", nbytes)
    n32 = nbytes // 4
    a = torch.randint(-2**31, 2**31 - 1, (n32 + 64,), dtype=torch.int32, device=DEV)
    b = torch.zeros_like(a)
    sp = torch.cuda.current_stream().cuda_stream
    assert rr.stream_copy_raw(a.data_ptr(), b.data_ptr(), nbytes, sp) == rr.RR_OK
    sink = torch.zeros(rr.stream_read_sink_bytes(nbytes) // 4, dtype=torch.int32, device=DEV)
    assert rr.stream_read_raw(a.data_ptr(), nbytes, sink.data_ptr(), sink.numel() * 4, sp) == 0
    c = torch.zeros_like(a)
    assert rr.stream_fill_raw(c.data_ptr(), nbytes, 0x1234ABCD, sp) == rr.RR_OK
    torch.cuda.synchronize()
    assert torch.equal(a[:n32], b[:n32]) and int(b[n32:].count_nonzero()) == 0
    def xor_all(t):
        t = t.to(torch.int64) & 0xFFFFFFFF
        while t.numel() > 1:
            if t.numel() % 2:
                t = torch.cat([t, torch.zeros(1, dtype=t.dtype, device=t.device)])
            t = t[0::2] ^ t[1::2]
        return int(t[0])
    assert xor_all(sink) == xor_all(a[:n32])
    assert bool((c[:n32] == 0x1234ABCD).all()) and int(c[n32:].count_nonzero()) == 0
    del a, b, c
    torch.cuda.empty_cache()


def test_stream_copy_binding():
    say("stream copy")
    a = torch.randn(1 << 20, device=DEV)
    b = torch.empty_like(a)
    rr.rr_stream_copy(a, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------- rows past on-chip capacity

# Aligned rows up to 2^23 elements stay on chip (split over up to 256 workgroups;
# rows that fill less than 9/10 of the largest plan, and softmax rows below 9/10 of
# 128 workgroups, read twice; aligned RMSNorm rows stay on chip at any fill, up to
# 2^23 elements and packed bf16 ones to 2^24, so their two-pass kernel is forced
# here); rows that are not 16-byte
# aligned hold at most 16 values on 1024 lanes of 16 workgroups on chip (262144
# elements) and go to the two-pass kernel past that.  The two-pass softmax splits
# fp32 rows of 5M elements over 64 workgroups and of 8M over 64.
LONG = [(3, 524289), (2, (1 << 22) + 8), (2, 1_000_003), (1, 5_000_000), (2, (1 << 23) + 8)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", LONG)
def test_long_rows_read_twice(M, N, dtype):
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    vec = N * (4 if dtype == "f32" else 2) % 16 == 0  # the 128-bit path needs 16-byte rows
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, M, N, code, vec)["path"] == 4
    say("long softmax", dtype, M, N)
    parity_softmax(_x(M, N, dtype, sigma=3.0), dtype, f"long softmax {dtype} {M}x{N}")
    on_chip = vec and 262144 < N <= 1 << (24 if dtype == "bf16" else 23)
    assert (rr.rr_plan_query(rr.RR_OP_RMSNORM, M, N, code, vec)["path"] == 4) != on_chip
    say("long rmsnorm", dtype, M, N)
    with forced(kind="long" if on_chip else None):
        assert rr.rr_plan_query(rr.RR_OP_RMSNORM, M, N, code, vec)["path"] == 4
        parity_rmsnorm(_x(M, N, dtype), _w(N, dtype), 1e-6, dtype, f"long rmsnorm {dtype} {M}x{N}")


ON_256 = [(3, 1 << 23), (2, 8_000_000), (3, 5_000_000), (4, 8_388_600)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", ON_256)
def test_rows_on_256_workgroups(M, N, dtype):
    """Rows of 5M to 8M elements on 64 values x 512 lanes x 256 workgroups (forced):
    one row group of every CU, the rows one after another through it (every slot set
    used), members past a short row's end holding nothing."""
    for op, run in (("softmax", lambda: parity_softmax(_x(M, N, dtype, sigma=3.0), dtype,
                                                       f"256 softmax {dtype} {M}x{N}")),
                    ("rmsnorm", lambda: parity_rmsnorm(_x(M, N, dtype), _w(N, dtype), 1e-6, dtype,
                                                       f"256 rmsnorm {dtype} {M}x{N}"))):
        with forced(64, 512, 256, kind="stream"):
            say("256 workgroups", op, dtype, M, N)
            run()


SPLIT_WIDE = [(3, 524288), (3, 524296), (2, 1 << 20), (5, 1_000_000), (40, 786432),
              (2, 1 << 21), (24, 1_500_000), (2, (1 << 21) + 8), (1, 3_000_000), (3, 1 << 22),
              (9, 3_500_000), (5, 3_800_000)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", SPLIT_WIDE)
def test_rows_split_over_many_workgroups(M, N, dtype):
    """Aligned rows from 2^19 to 2^22 elements: one read, 8 to 128 workgroups per row
    (bf16 RMSNorm packed, 8 to 64; 40 rows, or 9 rows on two row groups of 128, give
    each row group several rows, so every exchange slot set is used); softmax rows
    that fill less than 9/10 of 128 workgroups (bf16: of 64) read twice."""
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    for op in (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM):
        p = rr.rr_plan_query(op, M, N, code)
        if op == rr.RR_OP_SOFTMAX and 1 << 21 < N and 10 * N < 9 * (1 << 22):
            assert p["path"] == 4  # softmax on 128 workgroups: only from 9/10 full
            continue
        if (op == rr.RR_OP_SOFTMAX and dtype == "bf16" and 1 << 20 < N <= 1 << 21
                and 10 * N < 9 * (1 << 21)):
            assert p["path"] == 4  # bf16 softmax on 64 workgroups: only from 9/10 full
            continue
        assert p["path"] == 1 and p["groups_per_row"] >= 8, p
        assert p["vals_per_lane"] * p["lanes_per_row"] * p["groups_per_row"] >= N
    say("split32 softmax", dtype, M, N)
    parity_softmax(_x(M, N, dtype, sigma=3.0), dtype, f"split32 softmax {dtype} {M}x{N}")
    say("split32 rmsnorm", dtype, M, N)
    parity_rmsnorm(_x(M, N, dtype), _w(N, dtype), 1e-6, dtype, f"split32 rmsnorm {dtype} {M}x{N}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N", [(7, 1000), (33, 40000), (5, 16 * 16384 + 5), (70, 9)])
def test_long_row_kernel_forced_at_short_rows(M, N, dtype):
    """Tiles that do not fill a row group (members with no tile at all), ragged tails."""
    with forced(kind="long"):
        say("long forced softmax", dtype, M, N)
        parity_softmax(_x(M, N, dtype, sigma=2.0), dtype, f"long forced softmax {M}x{N}")
        say("long forced rmsnorm", dtype, M, N)
        parity_rmsnorm(_x(M, N, dtype), _w(N, dtype), 1e-6, dtype, f"long forced rmsnorm {M}x{N}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_long_rows_unaligned(dtype):
    M, N = 2, 600001
    x_np = _x(M, N, dtype, sigma=2.0)
    w_np = _w(N, dtype)
    xs = to_dev(np.concatenate([np.zeros(1, x_np.dtype), x_np.ravel()]), dtype)[1:].view(M, N)
    ys = torch.empty(M * N + 1, dtype=xs.dtype, device=DEV)[1:].view(M, N)
    wt = torch.empty(N + 1, dtype=xs.dtype, device=DEV)[1:]
    wt.copy_(to_dev(w_np, dtype))
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    say("long unaligned softmax", dtype)
    rr.rr_softmax_fwd(xs, ys, ws=rr.workspace(rr.RR_OP_SOFTMAX, M, N, code, DEV))
    torch.cuda.synchronize()
    check_out(from_dev(ys), oracle.softmax(x_np), dtype, "long unaligned softmax")
    say("long unaligned rmsnorm", dtype)
    rr.rr_rmsnorm_fwd(xs, wt, 1e-6, y=ys, ws=rr.workspace(rr.RR_OP_RMSNORM, M, N, code, DEV))
    torch.cuda.synchronize()
    check_out(from_dev(ys), oracle.rmsnorm(x_np, w_np, 1e-6), dtype, "long unaligned rmsnorm")


@pytest.mark.parametrize("kind", [None, "long"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_long_rows_many_rows_deterministic(dtype, kind):
    """Many rows of 600000 elements: split over 32 workgroups (default) or the
    two-pass kernel (forced)."""
    M, N = 200, 600000
    code = rr.RR_F32 if dtype == "f32" else rr.RR_BF16
    x_np = _x(M, N, dtype, sigma=2.0)
    x = to_dev(x_np, dtype)
    outs = []
    with forced(kind=kind):
        ws = rr.workspace(rr.RR_OP_SOFTMAX, M, N, code, DEV)
        for i in range(REPEATS):
            say("long rows repeat", kind, i, dtype)
            outs.append(rr.rr_softmax_fwd(x, ws=ws))
            torch.cuda.synchronize()
            assert int(ws.count_nonzero()) == 0
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    assert rr.rr_workspace_check(ws) == rr.RR_OK
    rows = np.arange(0, M, 23)
    check_out(from_dev(outs[0][torch.from_numpy(rows).to(DEV)]), oracle.softmax(x_np[rows]),
              dtype, "long rows sampled")
    s = outs[0].double().sum(dim=1)
    assert float((s - 1).abs().max()) < (1e-4 if dtype == "f32" else 5e-2)
