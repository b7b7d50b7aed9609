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


ALL = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
