"""Pins of the CPU oracle: facts fixed by mathematics, not by the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with the fact.  ``test_oracle_pins.py`` runs every pin on the
real oracle (all must hold) and on copies of ``oracle.c`` with a planted
mistake (each copy must fail at least one pin).

The facts:
- closed forms: constant rows, a row [B, 0, ..., 0], N = 1, a two-element row
  with large values (softmax is defined for any finite input);
- invariants: softmax rows sum to 1 and are unchanged, bit for bit, by adding
  an exactly representable constant; RMSNorm with eps = 0 is unchanged, bit
  for bit, by scaling the row by a power of two; the mean of (y/w)^2 is
  (Q/N)/(Q/N + eps); cross-entropy equals -log of the softmax entry at the
  label and lies in [0, ln N];
- brute force: the exact definition at 60 digits on tiny rows;
- a library routine: torch's float64 CPU softmax, rms_norm, logsumexp and
  cross_entropy(reduction='none') on small rows.

The backward functions (cross-entropy gradient, softmax backward, RMSNorm
backward) are pinned to the forward functions by calculus, not by their own
formulas:
- central differences of the (already pinned) forward functions, Richardson
  extrapolated over steps 2^-10 and 2^-9 taken on inputs that are multiples of
  2^-10, so every perturbed input is exact in fp32 and the remaining error is
  of order h^4;
- torch's float64 autograd (and its softmax backward from the output);
- invariants: a cross-entropy gradient row sums to zero, the RMSNorm input
  gradient satisfies sum_j x_j dx_j = r c (1 - r^2 Q / N), dw is additive
  over rows;
- closed forms: constant rows, one-hot and uniform softmax outputs.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np

import synth
from oracle import exact


def _rel(a, b):
    return abs(float(a) - float(b)) / max(abs(float(b)), 1e-300)


def _quantised_rows(rng, M, N, step=2.0**-10, lim=16.0):
    """fp32 rows whose entries are multiples of ``step`` in [-lim, lim]."""
    k = rng.integers(-int(lim / step), int(lim / step) + 1, size=(M, N))
    return (k * step).astype(np.float32)


# ------------------------------------------------------------------ softmax

def pin_softmax_rows_sum_to_one(o):
    for N in (1, 7, 256, 4097):
        x = synth.normal(5, N, sigma=3.0)
        y = o.softmax(x)
        assert np.all(np.abs(y.sum(axis=1) - 1.0) <= 1e-12), N
        assert np.all(y > 0)


def pin_softmax_shift_invariance_exact(o):
    rng = np.random.default_rng(1)
    x = _quantised_rows(rng, 6, 333)
    y = o.softmax(x)
    for c in (1.0, -7.0, 64.0):
        xs = (x + np.float32(c)).astype(np.float32)
        assert np.array_equal(xs - np.float32(c), x)  # the shift is exact in fp32
        assert np.array_equal(o.softmax(xs), y), c


def pin_softmax_constant_row(o):
    for N in (1, 2, 64, 1024, 65536):
        for c in (0.0, -3.5, 20.0):
            y = o.softmax(np.full((2, N), c, dtype=np.float32))
            assert np.all(y == 1.0 / N), (N, c)


def pin_softmax_spike_row_closed_form(o):
    # row [B, 0, ..., 0]: y_0 = 1 / (1 + (N-1) e^-B), y_j = e^-B / (1 + (N-1) e^-B)
    for N in (2, 5, 1000):
        for B in (0.75, 3.0, -2.5, 20.0):
            x = np.zeros((1, N), dtype=np.float32)
            x[0, 0] = B
            y = o.softmax(x)
            with localcontext() as ctx:
                ctx.prec = 50
                t = (-Decimal(B)).exp()
                d = 1 + (N - 1) * t
                y0, yj = 1 / d, t / d
            tol = (N + 4) * 2.0**-52  # a sequential double sum of N terms
            assert _rel(y[0, 0], y0) <= tol, (N, B)
            assert all(_rel(v, yj) <= tol for v in y[0, 1:]), (N, B)


def pin_softmax_large_values_stable(o):
    # softmax([a, a - 1]) = [1/(1+e^-1), e^-1/(1+e^-1)] for any finite a, and
    # softmax([a, 0]) = [1/(1+e^-a), e^-a/(1+e^-a)]
    for a in (1000.0, -1000.0, 3.0e38):
        x = np.array([[a, a - 1.0]], dtype=np.float32)
        if x[0, 0] - x[0, 1] != 1.0:
            x = np.array([[a, a]], dtype=np.float32)
            assert np.all(o.softmax(x) == 0.5)
            continue
        y = o.softmax(x)
        t = math.exp(-1.0)
        assert _rel(y[0, 0], 1 / (1 + t)) <= 1e-15 and _rel(y[0, 1], t / (1 + t)) <= 1e-15, a
    for a in (800.0, 90.0):
        with localcontext() as ctx:
            ctx.prec = 50
            t = (-Decimal(a)).exp()
            y0, y1 = 1 / (1 + t), t / (1 + t)
        # the large entry first, then last
        y = o.softmax(np.array([[a, 0.0], [0.0, a]], dtype=np.float32))
        assert np.all(np.isfinite(y))
        assert _rel(y[0, 0], y0) <= 1e-15 and _rel(y[0, 1], y1) <= 1e-13, a
        assert _rel(y[1, 1], y0) <= 1e-15 and _rel(y[1, 0], y1) <= 1e-13, a


def pin_softmax_brute_force(o):
    rng = np.random.default_rng(2)
    for N in (1, 3, 17, 64):
        x = (rng.standard_normal((3, N)) * 4).astype(np.float32)
        y = o.softmax(x)
        for i in range(3):
            ref = exact.softmax_row(x[i])
            assert max(_rel(a, b) for a, b in zip(y[i], ref)) <= 1e-14, N


def pin_softmax_matches_torch_f64(o):
    import torch

    x = synth.normal(9, 1000, sigma=3.0)
    ref = torch.softmax(torch.from_numpy(x).double(), dim=1).numpy()
    assert np.max(np.abs(o.softmax(x) - ref) / ref) <= 1e-13


def pin_softmax_bf16_decodes_exactly(o):
    # the same values given as bf16 bits and as fp32 give the same result
    xb = synth.normal(4, 200, dtype="bf16")
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(o.softmax(xb), o.softmax(xf))
    # known bit patterns: 0x3F80 = 1.0, 0x0000 = 0.0, 0xC000 = -2.0
    y = o.softmax(np.array([[0x3F80, 0x0000, 0xC000]], dtype=np.uint16))
    e1, e2 = math.exp(-1.0), math.exp(-3.0)
    d = 1 + e1 + e2
    assert all(_rel(a, b) <= 1e-15 for a, b in zip(y[0], (1 / d, e1 / d, e2 / d)))


def pin_softmax_rows_are_independent(o):
    x = synth.normal(12, 100)
    y = o.softmax(x)
    for i in (0, 5, 11):
        assert np.array_equal(o.softmax(x[i:i + 1]), y[i:i + 1])


# ------------------------------------------------------------------ RMSNorm

def pin_rmsnorm_constant_row(o):
    for N in (1, 3, 4096):
        for c in (1.0, -2.5, 0.125):
            for eps in (1e-6, 0.0, 0.5):
                w = synth.uniform(1, N, lo=0.5, hi=1.5).reshape(N)
                y = o.rmsnorm(np.full((2, N), c, dtype=np.float32), w, eps)
                e = float(np.float32(eps))
                ref = w.astype(np.float64) * c / math.sqrt(c * c + e)
                assert np.max(np.abs(y - ref) / np.abs(ref)) <= 4e-16, (N, c, eps)
                if eps == 0.0:
                    assert np.all(y == w.astype(np.float64) * math.copysign(1.0, c))


def pin_rmsnorm_power_of_two_scaling_exact(o):
    x = synth.normal(5, 1000)
    w = synth.uniform(1, 1000, lo=0.5, hi=1.5).reshape(1000)
    y = o.rmsnorm(x, w, 0.0)
    for k in (-7, 1, 12):
        assert np.array_equal(o.rmsnorm((x * np.float32(2.0**k)).astype(np.float32), w, 0.0), y)


def pin_rmsnorm_mean_square_identity(o):
    for eps in (1e-6, 0.25):
        for N in (1, 64, 4096):
            x = synth.normal(4, N, sigma=0.5)
            w = synth.uniform(1, N, lo=0.5, hi=1.5).reshape(N)
            y = o.rmsnorm(x, w, eps)
            q = np.array([math.fsum(float(v) * float(v) for v in row) for row in x]) / N
            e = float(np.float32(eps))
            lhs = np.mean((y / w.astype(np.float64)) ** 2, axis=1)
            assert np.all(np.abs(lhs - q / (q + e)) <= 1e-13), (eps, N)


def pin_rmsnorm_single_element(o):
    for v, wv in ((3.0, 1.25), (-0.5, 0.75), (2.0**-10, 1.5)):
        for eps in (1e-6, 1e-2):
            e = float(np.float32(eps))
            y = o.rmsnorm(np.array([[v]], dtype=np.float32), np.array([wv], dtype=np.float32), eps)
            ref = wv * v / math.sqrt(v * v + e)
            assert _rel(y[0, 0], ref) <= 4e-16


def pin_rmsnorm_brute_force(o):
    rng = np.random.default_rng(3)
    for N in (2, 13, 64):
        x = rng.standard_normal((3, N)).astype(np.float32)
        w = (rng.random(N) + 0.5).astype(np.float32)
        for eps in (1e-6, 0.3):
            y, rstd = o.rmsnorm(x, w, eps, want_rstd=True)
            for i in range(3):
                ref = exact.rmsnorm_row(x[i], w, np.float32(eps))
                assert max(_rel(a, b) for a, b in zip(y[i], ref)) <= 1e-14, (N, eps)
                ms = sum(float(v) ** 2 for v in x[i]) / N
                assert _rel(rstd[i], 1 / math.sqrt(ms + float(np.float32(eps)))) <= 1e-14


def pin_rmsnorm_matches_torch_f64(o):
    import torch

    x = synth.normal(7, 512)
    w = synth.uniform(1, 512, lo=0.5, hi=1.5).reshape(512)
    eps = 1e-6
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (512,),
                                       torch.from_numpy(w).double(),
                                       eps=float(np.float32(eps))).numpy()
    assert np.max(np.abs(o.rmsnorm(x, w, eps) - ref) / np.abs(ref)) <= 1e-13


def pin_rmsnorm_bf16_decodes_exactly(o):
    xb = synth.normal(3, 300, dtype="bf16")
    wb = synth.uniform(1, 300, lo=0.5, hi=1.5, dtype="bf16").reshape(300)
    dec = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(o.rmsnorm(xb, wb, 1e-6), o.rmsnorm(dec(xb), dec(wb), 1e-6))
    # [1.0, -2.0] with w = [1, 1], eps = 0: rms = sqrt(5/2)
    y = o.rmsnorm(np.array([[0x3F80, 0xC000]], dtype=np.uint16),
                  np.array([0x3F80, 0x3F80], dtype=np.uint16), 0.0)
    r = 1 / math.sqrt(2.5)
    assert _rel(y[0, 0], r) <= 4e-16 and _rel(y[0, 1], -2 * r) <= 4e-16


# ------------------------------------------------------------ cross-entropy

def pin_xent_is_minus_log_softmax(o):
    x = synth.normal(16, 1000, sigma=2.0)
    lab = synth.labels(16, 1000)
    loss, lse = o.cross_entropy(x, lab)
    y = o.softmax(x)
    assert np.max(np.abs(loss + np.log(y[np.arange(16), lab]))) <= 1e-12
    assert np.max(np.abs(lse - loss - x[np.arange(16), lab])) <= 1e-12


def pin_xent_constant_row(o):
    for N in (1, 2, 1000, 131072):
        for c in (0.0, 5.5, -20.0):
            loss, lse = o.cross_entropy(np.full((2, N), c, dtype=np.float32),
                                        np.array([0, N - 1], dtype=np.int32))
            assert np.all(np.abs(loss - math.log(N)) <= 1e-12), (N, c)
            assert np.all(np.abs(lse - (c + math.log(N))) <= 1e-12), (N, c)


def pin_xent_bounds(o):
    for N in (1, 10, 4096):
        x = synth.normal(8, N, sigma=2.0)
        lab = synth.labels(8, N)
        loss, lse = o.cross_entropy(x, lab)
        mx = x.max(axis=1).astype(np.float64)
        assert np.all(lse >= mx) and np.all(lse <= mx + math.log(N) + 1e-12)
        assert np.all(loss >= 0.0)
        if N == 1:
            assert np.all(loss == 0.0)


def pin_xent_label_is_used(o):
    # the label picks the row entry: loss differs by x_a - x_b between labels a, b
    x = synth.normal(1, 50, sigma=2.0)
    la, _ = o.cross_entropy(x, np.array([3], dtype=np.int32))
    lb, _ = o.cross_entropy(x, np.array([40], dtype=np.int32))
    assert abs((lb[0] - la[0]) - (float(x[0, 3]) - float(x[0, 40]))) <= 1e-13


def pin_xent_out_of_range_label_is_nan(o):
    x = synth.normal(4, 64)
    loss, lse = o.cross_entropy(x, np.array([-1, 64, 1 << 30, 5], dtype=np.int32))
    assert np.all(np.isnan(loss[:3])) and np.isfinite(loss[3])
    assert np.all(np.isfinite(lse))


def pin_xent_brute_force(o):
    rng = np.random.default_rng(4)
    for N in (1, 5, 64):
        x = (rng.standard_normal((3, N)) * 2).astype(np.float32)
        lab = rng.integers(0, N, size=3).astype(np.int32)
        loss, lse = o.cross_entropy(x, lab)
        for i in range(3):
            rl, rs = exact.cross_entropy_row(x[i], lab[i])
            assert abs(loss[i] - float(rl)) <= 1e-14 * max(1.0, abs(float(rl)))
            assert _rel(lse[i], rs) <= 1e-15


def pin_xent_matches_torch_f64(o):
    import torch

    x = synth.normal(10, 3000, sigma=2.0)
    lab = synth.labels(10, 3000)
    t = torch.from_numpy(x).double()
    ref_loss = torch.nn.functional.cross_entropy(t, torch.from_numpy(lab).long(),
                                                 reduction="none").numpy()
    ref_lse = torch.logsumexp(t, dim=1).numpy()
    loss, lse = o.cross_entropy(x, lab)
    assert np.max(np.abs(loss - ref_loss)) <= 1e-12
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def pin_xent_bf16_decodes_exactly(o):
    xb = synth.normal(3, 300, dtype="bf16", sigma=2.0)
    lab = synth.labels(3, 300)
    dec = (xb.astype(np.uint32) << 16).view(np.float32)
    a = o.cross_entropy(xb, lab)
    b = o.cross_entropy(dec, lab)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------- backward passes

_H = 2.0**-10


def _richardson(f, x, i, j, h=_H):
    """d f / d x[i, j] by central differences at h and 2h, extrapolated."""
    def d(step):
        xp = x.copy()
        xm = x.copy()
        xp[i, j] += np.float32(step)
        xm[i, j] -= np.float32(step)
        assert float(xp[i, j]) - float(x[i, j]) == step  # exact perturbation
        return (f(xp) - f(xm)) / (2.0 * step)
    return (4.0 * d(h) - d(2.0 * h)) / 3.0


def _dloss(M, seed_row=0):
    return synth.uniform(1, M, lo=0.5, hi=1.5, stream=synth.STREAM_DLOSS, row0=seed_row)[0]


def pin_xent_grad_forward_part_equals_forward(o):
    x = synth.normal(6, 777, sigma=2.0)
    lab = synth.labels(6, 777)
    loss, lse, _ = o.cross_entropy_grad(x, lab, _dloss(6))
    l2, s2 = o.cross_entropy(x, lab)
    assert np.array_equal(loss, l2) and np.array_equal(lse, s2)


def pin_xent_grad_finite_difference(o):
    rng = np.random.default_rng(11)
    x = _quantised_rows(rng, 3, 40, lim=4.0)
    lab = np.array([0, 17, 39], dtype=np.int32)
    g = np.array([1.0, 0.75, -2.5], dtype=np.float32)
    _, _, dx = o.cross_entropy_grad(x, lab, g)
    for i in range(3):
        for j in (0, 5, 17, 39, int(lab[i])):
            fd = _richardson(lambda z: o.cross_entropy(z, lab)[0][i], x, i, j)
            assert abs(dx[i, j] - float(g[i]) * fd) <= 1e-9, (i, j)


def pin_xent_grad_rows_sum_to_zero(o):
    for N in (1, 2, 1000):
        x = synth.normal(5, N, sigma=2.0)
        lab = synth.labels(5, N)
        g = _dloss(5)
        _, _, dx = o.cross_entropy_grad(x, lab, g)
        assert np.all(np.abs(dx.sum(axis=1)) <= 1e-14 * N), N
        # the label entry is the only non-positive one (for a positive dloss)
        assert np.all(dx[np.arange(5), lab] <= 0.0)
        off = dx.copy()
        off[np.arange(5), lab] = 0.0
        assert np.all(off >= 0.0)


def pin_xent_grad_constant_row(o):
    for N in (1, 4, 1000):
        x = np.full((2, N), 3.25, dtype=np.float32)
        lab = np.array([0, N - 1], dtype=np.int32)
        g = np.array([1.0, 0.5], dtype=np.float32)
        _, _, dx = o.cross_entropy_grad(x, lab, g)
        for i in range(2):
            want = np.full(N, 1.0 / N)
            want[lab[i]] -= 1.0
            assert np.max(np.abs(dx[i] - want * float(g[i]))) <= 1e-15, N


def pin_xent_grad_matches_torch_f64(o):
    import torch

    x = synth.normal(8, 2000, sigma=2.0)
    lab = synth.labels(8, 2000)
    g = _dloss(8)
    t = torch.from_numpy(x).double().requires_grad_(True)
    loss = torch.nn.functional.cross_entropy(t, torch.from_numpy(lab).long(), reduction="none")
    loss.backward(torch.from_numpy(g).double())
    _, _, dx = o.cross_entropy_grad(x, lab, g)
    assert np.max(np.abs(dx - t.grad.numpy())) <= 1e-15


def pin_xent_grad_invalid_label_row_is_nan(o):
    x = synth.normal(3, 64)
    lab = np.array([-1, 64, 5], dtype=np.int32)
    loss, lse, dx = o.cross_entropy_grad(x, lab, _dloss(3))
    assert np.all(np.isnan(loss[:2])) and np.isfinite(loss[2])
    assert np.all(np.isnan(dx[:2])) and np.all(np.isfinite(dx[2]))
    assert np.all(np.isfinite(lse))


def pin_xent_grad_bf16_decodes_exactly(o):
    xb = synth.normal(3, 300, dtype="bf16", sigma=2.0)
    lab = synth.labels(3, 300)
    dec = (xb.astype(np.uint32) << 16).view(np.float32)
    g = _dloss(3)
    a = o.cross_entropy_grad(xb, lab, g)
    b = o.cross_entropy_grad(dec, lab, g)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def pin_softmax_bwd_matches_torch_f64(o):
    import torch

    for dt in ("f32", "bf16"):
        y = o.softmax(synth.normal(6, 1500, sigma=2.0, dtype=dt))
        y = y.astype(np.float32) if dt == "f32" else synth.f32_to_bf16(y.astype(np.float32))
        dy = synth.normal(6, 1500, dtype=dt, stream=synth.STREAM_DY)
        dec = (lambda a: a.astype(np.float64) if dt == "f32"
               else (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        ref = torch._softmax_backward_data(torch.from_numpy(dec(dy)), torch.from_numpy(dec(y)), 1,
                                           torch.float64).numpy()
        dx = o.softmax_backward(y, dy)
        scale = np.abs(dec(y)) * (np.abs(dec(dy)) + np.abs(dec(y) * dec(dy)).sum(1, keepdims=True))
        assert np.all(np.abs(dx - ref) <= 1e-13 * scale + 1e-300), dt


def pin_softmax_bwd_finite_difference(o):
    rng = np.random.default_rng(12)
    x = _quantised_rows(rng, 2, 30, lim=4.0)
    dy = (rng.standard_normal((2, 30))).astype(np.float32)
    y = o.softmax(x).astype(np.float32)
    dx = o.softmax_backward(y, dy)
    for i in range(2):
        for j in (0, 7, 29):
            fd = _richardson(lambda z: float(np.dot(o.softmax(z)[i], dy[i].astype(np.float64))),
                             x, i, j)
            # y enters the backward rounded to fp32: about 2^-24 of each term
            tol = 1e-6 * float(y[i, j]) * (abs(float(dy[i, j])) + float(np.abs(y[i] * dy[i]).sum()))
            assert abs(dx[i, j] - fd) <= tol + 1e-12, (i, j)


def pin_softmax_bwd_closed_forms(o):
    # one-hot output: no gradient at all
    y = np.zeros((1, 50), dtype=np.float32)
    y[0, 13] = 1.0
    dy = synth.normal(1, 50, stream=synth.STREAM_DY)
    assert np.all(o.softmax_backward(y, dy) == 0.0)
    # uniform output 1/N (N a power of two, exact): dx_j = (dy_j - mean(dy)) / N
    N = 64
    y = np.full((1, N), 1.0 / N, dtype=np.float32)
    dy = synth.normal(1, N, stream=synth.STREAM_DY)
    want = (dy[0].astype(np.float64) - dy[0].astype(np.float64).mean()) / N
    assert np.max(np.abs(o.softmax_backward(y, dy)[0] - want)) <= 1e-17
    # a constant upstream gradient has no effect on a normalised output
    y = o.softmax(synth.normal(2, 200)).astype(np.float32)
    dx = o.softmax_backward(y, np.full((2, 200), 0.75, dtype=np.float32))
    s = y.astype(np.float64).sum(axis=1, keepdims=True)
    assert np.max(np.abs(dx - 0.75 * y * (1.0 - s))) <= 1e-16


def pin_softmax_bwd_bf16_decodes_exactly(o):
    yb = synth.uniform(3, 256, lo=0.0, hi=0.01, dtype="bf16")
    db = synth.normal(3, 256, dtype="bf16", stream=synth.STREAM_DY)
    dec = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(o.softmax_backward(yb, db), o.softmax_backward(dec(yb), dec(db)))


def _rms_case(M, N, dtype="f32"):
    x = synth.normal(M, N, dtype=dtype)
    w = synth.uniform(1, N, lo=0.5, hi=1.5, dtype=dtype)[0]
    dy = synth.normal(M, N, dtype=dtype, stream=synth.STREAM_DY)
    return x, w, dy


def pin_rmsnorm_bwd_finite_difference(o):
    rng = np.random.default_rng(13)
    x = _quantised_rows(rng, 2, 24, lim=4.0)
    w = _quantised_rows(rng, 1, 24, lim=2.0)[0]
    dy = rng.standard_normal((2, 24)).astype(np.float32)
    eps = 1e-3
    _, r = o.rmsnorm(x, w, eps, want_rstd=True)
    dx, dw = o.rmsnorm_backward(x, w, dy, r.astype(np.float32))
    for i in range(2):
        for j in (0, 11, 23):
            fd = _richardson(lambda z: float(np.dot(o.rmsnorm(z, w, eps)[i],
                                                    dy[i].astype(np.float64))), x, i, j)
            # rstd enters the backward rounded to fp32
            assert abs(dx[i, j] - fd) <= 2e-6 * (abs(fd) + 1e-3), (i, j)
    wm = w[None, :].copy()
    for j in (0, 9, 23):
        fd = _richardson(lambda z: float(np.sum(o.rmsnorm(x, z[0], eps) * dy.astype(np.float64))),
                         wm, 0, j)
        assert abs(dw[j] - fd) <= 2e-6 * (abs(fd) + 1e-3), j


def pin_rmsnorm_bwd_matches_torch_f64_exact_rstd(o):
    """eps is chosen per row so that the exact r is an fp32 value: the backward
    then sees exactly the r of the forward torch differentiates."""
    import torch

    M, N = 4, 500
    x, w, dy = _rms_case(M, N)
    q = (x.astype(np.float64) ** 2).mean(axis=1)
    for i in range(M):
        r = np.float32(0.9 / math.sqrt(q[i]))
        eps_i = 1.0 / float(r) ** 2 - q[i]
        assert eps_i > 0
        t = torch.from_numpy(x[i:i + 1].astype(np.float64)).requires_grad_(True)
        tw = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
        y = torch.nn.functional.rms_norm(t, (N,), tw, eps=eps_i)
        y.backward(torch.from_numpy(dy[i:i + 1].astype(np.float64)))
        dx, dw = o.rmsnorm_backward(x[i:i + 1], w, dy[i:i + 1], np.array([r], dtype=np.float32))
        assert np.max(np.abs(dx - t.grad.numpy())) <= 1e-12 * np.max(np.abs(dx)), i
        assert np.max(np.abs(dw - tw.grad.numpy())) <= 1e-12 * np.max(np.abs(dw)), i


def pin_rmsnorm_bwd_orthogonality_identity(o):
    """sum_j x_j dx_j = r c (1 - r^2 Q / N) for any r; with the exact forward r
    the bracket is r^2 eps, and with eps = 0 the gradient is orthogonal to x."""
    x, w, dy = _rms_case(5, 3000)
    _, r = o.rmsnorm(x, w, 0.0, want_rstd=True)
    r32 = r.astype(np.float32)
    dx, _ = o.rmsnorm_backward(x, w, dy, r32)
    xd = x.astype(np.float64)
    c = (dy.astype(np.float64) * w.astype(np.float64) * xd).sum(axis=1)
    q = (xd * xd).sum(axis=1)
    rr = r32.astype(np.float64)
    lhs = (xd * dx).sum(axis=1)
    rhs = rr * c * (1.0 - rr * rr * q / 3000)
    scale = np.abs(xd * dx).sum(axis=1) + np.abs(rr * c)
    assert np.all(np.abs(lhs - rhs) <= 1e-13 * scale)


def pin_rmsnorm_bwd_dw_adds_over_rows(o):
    x, w, dy = _rms_case(6, 700)
    _, r = o.rmsnorm(x, w, 1e-6, want_rstd=True)
    r32 = r.astype(np.float32)
    _, dw = o.rmsnorm_backward(x, w, dy, r32)
    parts = sum(o.rmsnorm_backward(x[i:i + 1], w, dy[i:i + 1], r32[i:i + 1])[1] for i in range(6))
    assert np.max(np.abs(dw - parts)) <= 1e-13 * np.max(np.abs(dw))
    # and doubling a row's upstream gradient doubles its share
    dy2 = dy.copy()
    dy2[0] *= 2
    _, dw2 = o.rmsnorm_backward(x, w, dy2, r32)
    one = o.rmsnorm_backward(x[:1], w, dy[:1], r32[:1])[1]
    assert np.max(np.abs(dw2 - dw - one)) <= 1e-12 * np.max(np.abs(dw))


def pin_rmsnorm_bwd_bf16_decodes_exactly(o):
    x, w, dy = _rms_case(3, 256, "bf16")
    dec = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    r = np.array([0.5, 1.0, 0.75], dtype=np.float32)
    a = o.rmsnorm_backward(x, w, dy, r)
    b = o.rmsnorm_backward(dec(x), dec(w), dec(dy), r)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


ALL = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
