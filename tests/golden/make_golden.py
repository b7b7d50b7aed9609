"""Writes ``tiny_cases.json``: tiny hand-built rows and their exact results.

The source pages print no worked example for any of the three operators, so
the stored values here are not quoted from them.  They are the textbook
definitions evaluated at 60 significant digits by ``oracle/exact.py`` (the
arbitrary-precision part of the oracle); this script calls nothing else.
Inputs are written as exact hexadecimal floats (fp32) or bf16 bit patterns.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from oracle import exact  # noqa: E402

DIGITS = 25


def f32(vals):
    return [float(np.float32(v)).hex() for v in vals]


def bf16_value(bits):
    return float((np.array([bits], dtype=np.uint32) << 16).view(np.float32)[0])


def fmt(d):
    return format(d, f".{DIGITS}e")


def main():
    cases = []

    def softmax_case(name, dtype, rows):
        if dtype == "f32":
            xs = [[float(np.float32(v)) for v in r] for r in rows]
            enc = [f32(r) for r in rows]
        else:
            xs = [[bf16_value(b) for b in r] for r in rows]
            enc = [[f"{b:04x}" for b in r] for r in rows]
        y = [[fmt(v) for v in exact.softmax_row(r)] for r in xs]
        cases.append({"name": name, "op": "softmax", "dtype": dtype, "x": enc, "y": y})

    def rmsnorm_case(name, dtype, rows, w, eps):
        if dtype == "f32":
            xs = [[float(np.float32(v)) for v in r] for r in rows]
            ws = [float(np.float32(v)) for v in w]
            enc, wenc = [f32(r) for r in rows], f32(w)
        else:
            xs = [[bf16_value(b) for b in r] for r in rows]
            ws = [bf16_value(b) for b in w]
            enc = [[f"{b:04x}" for b in r] for r in rows]
            wenc = [f"{b:04x}" for b in w]
        y = [[fmt(v) for v in exact.rmsnorm_row(r, ws, float(np.float32(eps)))] for r in xs]
        cases.append({"name": name, "op": "rmsnorm", "dtype": dtype, "x": enc, "w": wenc,
                      "eps": eps, "y": y})

    def xent_case(name, rows, labels):
        xs = [[float(np.float32(v)) for v in r] for r in rows]
        res = [exact.cross_entropy_row(r, t) for r, t in zip(xs, labels)]
        cases.append({"name": name, "op": "xent", "dtype": "f32", "x": [f32(r) for r in rows],
                      "labels": labels, "loss": [fmt(l) for l, _ in res],
                      "lse": [fmt(s) for _, s in res]})

    def xent_grad_case(name, rows, labels, dloss):
        xs = [[float(np.float32(v)) for v in r] for r in rows]
        gs = [float(np.float32(g)) for g in dloss]
        dx = [[fmt(v) for v in exact.cross_entropy_grad_row(r, t, g)]
              for r, t, g in zip(xs, labels, gs)]
        res = [exact.cross_entropy_row(r, t) for r, t in zip(xs, labels)]
        cases.append({"name": name, "op": "xent_grad", "dtype": "f32",
                      "x": [f32(r) for r in rows], "labels": labels, "dloss": f32(dloss),
                      "loss": [fmt(l) for l, _ in res], "lse": [fmt(s) for _, s in res],
                      "dx": dx})

    def rmsnorm_bwd_case(name, rows, w, dy, rstd):
        """rstd is an fp32 value per row; eps is set per row (at 60 digits) so
        that the forward's exact r is that value, and is stored for reference."""
        from decimal import Decimal, localcontext
        xs = [[float(np.float32(v)) for v in r] for r in rows]
        ws = [float(np.float32(v)) for v in w]
        gs = [[float(np.float32(v)) for v in r] for r in dy]
        dxs, dws, epss = [], [], []
        dw_tot = None
        with localcontext() as ctx:
            ctx.prec = exact.PREC
            for r_x, r_g, r32 in zip(xs, gs, rstd):
                r = Decimal(float(np.float32(r32)))
                ms = sum((Decimal(v) * Decimal(v) for v in r_x), Decimal(0)) / len(r_x)
                eps = 1 / (r * r) - ms
                assert eps > 0
                dx, dw = exact.rmsnorm_backward_row(r_x, ws, r_g, eps)
                dxs.append([fmt(v) for v in dx])
                dw_tot = dw if dw_tot is None else [a + b for a, b in zip(dw_tot, dw)]
                epss.append(fmt(eps))
        cases.append({"name": name, "op": "rmsnorm_bwd", "dtype": "f32",
                      "x": [f32(r) for r in rows], "w": f32(w), "dy": [f32(r) for r in dy],
                      "rstd": f32(rstd), "eps_for_rstd": epss, "dx": dxs,
                      "dw": [fmt(v) for v in dw_tot]})

    softmax_case("ramp_and_spike", "f32", [[0, 1, 2, 3], [20, 0, 0, 0], [-1.5, -1.5, 2.25, 0.5]])
    softmax_case("single_element", "f32", [[5.0]])
    softmax_case("bf16_patterns", "bf16", [[0x3F80, 0xC000, 0x3F00, 0x0000, 0x4120]])
    rmsnorm_case("small_rows", "f32", [[1, 2, 3, 4], [-0.5] * 4], [1.0, 0.5, 1.5, 1.25], 1e-6)
    rmsnorm_case("bf16_patterns", "bf16", [[0x3F80, 0xC000, 0x3F00, 0x4120]],
                 [0x3F80, 0x3FC0, 0x3F40, 0x3F80], 1e-6)
    xent_case("ramp_rows", [[0, 1, 2, 3], [2.5, 2.5, 2.5, 2.5], [10, -10, 0, 5]], [2, 0, 1])
    xent_grad_case("ramp_rows_grad", [[0, 1, 2, 3], [2.5, 2.5, 2.5, 2.5], [10, -10, 0, 5]],
                   [2, 0, 1], [1.0, 0.25, -3.0])
    rmsnorm_bwd_case("small_rows_bwd", [[1, 2, 3, 4], [-0.5, 0.25, 1.5, -2.0]],
                     [1.0, 0.5, 1.5, 1.25], [[0.5, -1.0, 2.0, 0.25], [1.0, 1.0, -1.0, 0.5]],
                     [0.3125, 0.75])

    doc = {
        "citation": "No worked example is printed on the source pages (QuACK article "
                    "无需CUDA代码，给H100加速33%-50%); these are the textbook definitions of "
                    "softmax, RMSNorm (eps inside the root, weight, no bias) and per-row "
                    "cross-entropy, evaluated at 60 digits by oracle/exact.py; the gradient "
                    "cases are central differences of those definitions at 60 digits.",
        "cases": cases,
    }
    with open(os.path.join(HERE, "tiny_cases.json"), "w") as f:
        json.dump(doc, f, indent=1, ensure_ascii=False)
        f.write("\n")


if __name__ == "__main__":
    main()
