"""Arbitrary-precision brute force for tiny rows (an independent pin of ``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Pure-Python loops over ``decimal.Decimal`` at 60
significant digits, so it is meant for rows of at most a few hundred
elements.  Every input value is taken exactly (an fp32 or bf16 value is a
dyadic rational, which ``Decimal(float)`` represents without rounding); exp,
ln and sqrt are the decimal module's correctly rounded functions.  The
definitions are the textbook ones (see ``oracle.c``), but this file computes
them with no max subtraction: softmax_j = exp(x_j) / sum_k exp(x_k), so the
row-max step of the double oracle is checked rather than repeated.

The gradients are not written from their closed forms at all: each is the
central difference of a forward function above, (f(x + h) - f(x - h)) / 2h
with h = 10^-20 at 60 digits, whose error (of order h^2 times the third
derivative, plus 10^-40 of cancellation) is far below the 25 digits kept.
"""
from __future__ import annotations

from decimal import Decimal, localcontext

PREC = 60


def _dec(v) -> Decimal:
    return Decimal(float(v))


def softmax_row(row):
    with localcontext() as ctx:
        ctx.prec = PREC
        ex = [_dec(v).exp() for v in row]
        s = sum(ex, Decimal(0))
        return [e / s for e in ex]


def rmsnorm_row(row, w, eps):
    with localcontext() as ctx:
        ctx.prec = PREC
        xs = [_dec(v) for v in row]
        n = Decimal(len(xs))
        ms = sum((v * v for v in xs), Decimal(0)) / n
        denom = (ms + _dec(eps)).sqrt()
        return [v * _dec(wj) / denom for v, wj in zip(xs, w)]


def logsumexp_row(row):
    with localcontext() as ctx:
        ctx.prec = PREC
        return sum((_dec(v).exp() for v in row), Decimal(0)).ln()


def cross_entropy_row(row, label):
    """(loss, lse) for one row; loss is None for a label outside [0, N)."""
    lse = logsumexp_row(row)
    if not 0 <= int(label) < len(row):
        return None, lse
    with localcontext() as ctx:
        ctx.prec = PREC
        return lse - _dec(row[int(label)]), lse


_FD_STEP = Decimal("1e-20")


def _central(f, xs, j):
    """d f / d xs[j] by a central difference on Decimal inputs."""
    xp = list(xs)
    xm = list(xs)
    xp[j] = xs[j] + _FD_STEP
    xm[j] = xs[j] - _FD_STEP
    return (f(xp) - f(xm)) / (2 * _FD_STEP)


def _lse_dec(xs):
    return sum((v.exp() for v in xs), Decimal(0)).ln()


def cross_entropy_grad_row(row, label, dloss):
    """d(loss)/dx_j * dloss for one row (label in range)."""
    with localcontext() as ctx:
        ctx.prec = PREC
        xs = [_dec(v) for v in row]
        t = int(label)
        loss = lambda z: _lse_dec(z) - z[t]
        g = _dec(dloss)
        return [_central(loss, xs, j) * g for j in range(len(xs))]


def rmsnorm_backward_row(row, w, dy, eps):
    """(dx, dw share) of one row: derivatives of sum_j dy_j * y_j(x, w), with
    y the RMSNorm of the row (eps a Decimal, so the caller controls r)."""
    with localcontext() as ctx:
        ctx.prec = PREC
        xs = [_dec(v) for v in row]
        ws = [_dec(v) for v in w]
        gs = [_dec(v) for v in dy]
        n = Decimal(len(xs))

        def f(x, wv):
            ms = sum((v * v for v in x), Decimal(0)) / n
            r = 1 / (ms + eps).sqrt()
            return sum((gj * xj * r * wj for gj, xj, wj in zip(gs, x, wv)), Decimal(0))

        dx = [_central(lambda z: f(z, ws), xs, j) for j in range(len(xs))]
        dw = [_central(lambda z: f(xs, z), ws, j) for j in range(len(ws))]
        return dx, dw
