"""Arbitrary-precision brute force for tiny rows (an independent pin of ``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Pure-Python loops over ``decimal.Decimal`` at 60
significant digits, so it is meant for rows of at most a few hundred
elements.  Every input value is taken exactly (an fp32 or bf16 value is a
dyadic rational, which ``Decimal(float)`` represents without rounding); exp,
ln and sqrt are the decimal module's correctly rounded functions.  The
definitions are the textbook ones (see ``oracle.c``), but this file computes
them with no max subtraction: softmax_j = exp(x_j) / sum_k exp(x_k), so the
row-max step of the double oracle is checked rather than repeated.
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
