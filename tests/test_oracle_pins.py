"""The oracle against its pins, and planted mistakes that the pins must catch.

Every pin in ``_pins.py`` must hold for ``oracle/oracle.c``.  Then, for each
plausible mistake (a dropped term, a wrong sign or index, a swapped operand,
a wrong decode), a copy of ``oracle.c`` with that one mistake is compiled on
the CPU and at least one pin must fail on it.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from oracle import compile_library

from _pins import ALL

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_cases.json")


@pytest.mark.parametrize("pin", ALL, ids=[p.__name__ for p in ALL])
def test_pin_holds(pin, orc):
    pin(orc)


# (id, function the mistake goes in, exact text, replacement)
MUTANTS = [
    ("softmax_no_max_subtraction", "oracle_softmax",
     "exp(load_elem(x, dtype, row + j) - m)", "exp(load_elem(x, dtype, row + j))"),
    ("softmax_min_instead_of_max", "oracle_softmax",
     "if (v > m || isnan(v)) m = v;", "if (j == 0 || v < m) m = v;"),
    ("softmax_first_element_as_max", "oracle_softmax",
     "if (v > m || isnan(v)) m = v;", "if (j == 0) m = v;"),
    ("softmax_max_skips_last", "oracle_softmax",
     "for (int64_t j = 0; j < N; ++j) {\n            double v", "for (int64_t j = 0; j < N - 1; ++j) {\n            double v"),
    ("softmax_divides_by_N", "oracle_softmax", "y[row + j] / S", "y[row + j] / (double)N"),
    ("softmax_row_offset_dropped", "oracle_softmax", "y[row + j] = e;", "y[j] = e;"),
    ("softmax_sum_skips_first", "oracle_softmax", "S += e;", "if (j > 0) S += e;"),
    ("rmsnorm_no_eps", "oracle_rmsnorm", "Q / (double)N + e", "Q / (double)N"),
    ("rmsnorm_eps_outside_root", "oracle_rmsnorm", "sqrt(Q / (double)N + e)", "(sqrt(Q / (double)N) + e)"),
    ("rmsnorm_sum_not_mean", "oracle_rmsnorm", "Q / (double)N + e", "Q + e"),
    ("rmsnorm_mean_over_N_minus_1", "oracle_rmsnorm", "Q / (double)N + e", "Q / (double)(N - 1) + e"),
    ("rmsnorm_not_squared", "oracle_rmsnorm", "Q += v * v;", "Q += v;"),
    ("rmsnorm_weight_index", "oracle_rmsnorm", "load_elem(w, dtype, j)", "load_elem(w, dtype, 0)"),
    ("rmsnorm_no_weight", "oracle_rmsnorm", " * r * load_elem(w, dtype, j)", " * r"),
    ("rmsnorm_sqrt_not_rsqrt", "oracle_rmsnorm", "1.0 / sqrt(", "sqrt("),
    ("xent_loss_sign", "oracle_cross_entropy", "l - load_elem(x, dtype, row + t)",
     "l + load_elem(x, dtype, row + t)"),
    ("xent_loss_operands_swapped", "oracle_cross_entropy", "l - load_elem(x, dtype, row + t)",
     "load_elem(x, dtype, row + t) - l"),
    ("xent_lse_missing_max", "oracle_cross_entropy", "double l = m + log(S);", "double l = log(S);"),
    ("xent_label_row_offset", "oracle_cross_entropy", "load_elem(x, dtype, row + t)",
     "load_elem(x, dtype, t)"),
    ("xent_label_off_by_one", "oracle_cross_entropy", "load_elem(x, dtype, row + t)",
     "load_elem(x, dtype, row + (t + 1) % N)"),
    ("xent_no_range_check", "oracle_cross_entropy", "(t >= 0 && (int64_t)t < N) ?",
     "(t >= 0) ?"),
    ("xent_grad_onehot_sign", "oracle_cross_entropy_grad", "(p - onehot) * g", "(p + onehot) * g"),
    ("xent_grad_no_dloss", "oracle_cross_entropy_grad", "(p - onehot) * g", "(p - onehot)"),
    ("xent_grad_onehot_index", "oracle_cross_entropy_grad", "(j == (int64_t)t)",
     "(j == (int64_t)t + 1)"),
    ("xent_grad_p_missing_max", "oracle_cross_entropy_grad",
     "double p = exp(load_elem(x, dtype, row + j) - m) / S;",
     "double p = exp(load_elem(x, dtype, row + j)) / S;"),
    ("xent_grad_p_not_normalised", "oracle_cross_entropy_grad",
     "double p = exp(load_elem(x, dtype, row + j) - m) / S;",
     "double p = exp(load_elem(x, dtype, row + j) - m);"),
    ("xent_grad_lse_missing_max", "oracle_cross_entropy_grad", "double l = m + log(S);",
     "double l = log(S);"),
    ("xent_grad_invalid_label_not_nan", "oracle_cross_entropy_grad",
     "dx[row + j] = ok ? (p - onehot) * g : NAN;", "dx[row + j] = (p - onehot) * g;"),
    ("xent_grad_dloss_of_wrong_row", "oracle_cross_entropy_grad", "double g = (double)dloss[i];",
     "double g = (double)dloss[0];"),
    ("softmax_bwd_no_c", "oracle_softmax_backward", "* (load_elem(dy, dtype, row + j) - c)",
     "* load_elem(dy, dtype, row + j)"),
    ("softmax_bwd_c_sign", "oracle_softmax_backward", "(load_elem(dy, dtype, row + j) - c)",
     "(load_elem(dy, dtype, row + j) + c)"),
    ("softmax_bwd_c_without_y", "oracle_softmax_backward",
     "c += load_elem(y, dtype, row + k) * load_elem(dy, dtype, row + k);",
     "c += load_elem(dy, dtype, row + k);"),
    ("softmax_bwd_y_index", "oracle_softmax_backward", "dx[row + j] = load_elem(y, dtype, row + j)",
     "dx[row + j] = load_elem(y, dtype, row + (j + 1) % N)"),
    ("softmax_bwd_c_skips_last", "oracle_softmax_backward", "for (int64_t k = 0; k < N; ++k)",
     "for (int64_t k = 0; k < N - 1; ++k)"),
    ("rmsnorm_bwd_r_squared", "oracle_rmsnorm_backward", "r * r * r * xj", "r * r * xj"),
    ("rmsnorm_bwd_N_minus_1", "oracle_rmsnorm_backward", "c / (double)N", "c / (double)(N - 1)"),
    ("rmsnorm_bwd_c_without_weight", "oracle_rmsnorm_backward",
     "load_elem(dy, dtype, row + k) * load_elem(w, dtype, k) * load_elem(x, dtype, row + k)",
     "load_elem(dy, dtype, row + k) * load_elem(x, dtype, row + k)"),
    ("rmsnorm_bwd_sign", "oracle_rmsnorm_backward", "* gj - r * r * r", "* gj + r * r * r"),
    ("rmsnorm_bwd_dx_without_weight", "oracle_rmsnorm_backward", "r * load_elem(w, dtype, j) * gj",
     "r * gj"),
    ("rmsnorm_bwd_dw_without_r", "oracle_rmsnorm_backward", "dw[j] += gj * xj * r;",
     "dw[j] += gj * xj;"),
    ("rmsnorm_bwd_dw_overwritten", "oracle_rmsnorm_backward", "dw[j] += gj * xj * r;",
     "dw[j] = gj * xj * r;"),
    ("rmsnorm_bwd_dw_uses_weight", "oracle_rmsnorm_backward", "dw[j] += gj * xj * r;",
     "dw[j] += gj * xj * r * load_elem(w, dtype, j);"),
    ("bf16_decode_shift", "load_elem", "<< 16", "<< 15"),
    ("bf16_decoded_as_f32_path", "load_elem", "if (dtype == ORACLE_F32)", "if (dtype != ORACLE_F32)"),
]


def _mutate(src, func, old, new):
    start = src.index(func + "(")
    end = src.index("\n}\n", start)
    body = src[start:end]
    assert body.count(old) == 1, f"mutation text must occur once in {func}: {old!r}"
    return src[:start] + body.replace(old, new) + src[end:]


_RUNNER = """
import sys
sys.path[:0] = {paths!r}
import numpy as np
from oracle import Oracle, bind
from _pins import ALL
o = Oracle(bind({lib!r}))
for pin in ALL:
    try:
        with np.errstate(all="ignore"):
            pin(o)
    except Exception as exc:
        print("caught by", pin.__name__, type(exc).__name__)
        sys.exit(0)
print("no pin failed")
sys.exit(3)
"""


@pytest.mark.parametrize("mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(mut, tmp_path):
    """Each mutant runs in a child process: a mutant that reads out of bounds
    and crashes has been caught as well."""
    name, func, old, new = mut
    src = open(ORACLE_SRC).read()
    path = tmp_path / f"{name}.c"
    path.write_text(_mutate(src, func, old, new))
    lib = compile_library(str(path), str(tmp_path / f"lib{name}.so"))
    here = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER.format(paths=[here, os.path.dirname(here)], lib=lib)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=600)
    assert res.returncode != 3, f"no pin catches the planted mistake {name}: {res.stdout}"
    assert res.returncode == 0 or res.returncode < 0, res.stderr[-2000:]


def test_mutations_apply_to_the_real_source():
    src = open(ORACLE_SRC).read()
    for name, func, old, new in MUTANTS:
        assert _mutate(src, func, old, new) != src, name


# ------------------------------------------------------------ golden cases

def _decode_case(c):
    if c["dtype"] == "f32":
        x = np.array([[float.fromhex(v) for v in row] for row in c["x"]], dtype=np.float32)
        w = (np.array([float.fromhex(v) for v in c["w"]], dtype=np.float32)
             if "w" in c else None)
    else:
        x = np.array([[int(v, 16) for v in row] for row in c["x"]], dtype=np.uint16)
        w = np.array([int(v, 16) for v in c["w"]], dtype=np.uint16) if "w" in c else None
    return x, w


def test_oracle_matches_golden_cases(orc):
    data = json.load(open(GOLDEN))
    assert data["cases"]
    for c in data["cases"]:
        x, w = _decode_case(c)
        if c["op"] == "softmax":
            got = orc.softmax(x)
            exp = np.array([[float(v) for v in row] for row in c["y"]])
            assert np.max(np.abs(got - exp) / np.abs(exp)) <= 1e-14, c["name"]
        elif c["op"] == "rmsnorm":
            got = orc.rmsnorm(x, w, c["eps"])
            exp = np.array([[float(v) for v in row] for row in c["y"]])
            assert np.max(np.abs(got - exp) / np.abs(exp)) <= 1e-14, c["name"]
        elif c["op"] == "xent":
            loss, lse = orc.cross_entropy(x, np.array(c["labels"], dtype=np.int32))
            assert np.max(np.abs(lse - np.array([float(v) for v in c["lse"]]))) <= 1e-13, c["name"]
            assert np.max(np.abs(loss - np.array([float(v) for v in c["loss"]]))) <= 1e-13, c["name"]
        elif c["op"] == "xent_grad":
            g = np.array([float.fromhex(v) for v in c["dloss"]], dtype=np.float32)
            loss, lse, dx = orc.cross_entropy_grad(x, np.array(c["labels"], dtype=np.int32), g)
            assert np.max(np.abs(loss - np.array([float(v) for v in c["loss"]]))) <= 1e-13, c["name"]
            exp = np.array([[float(v) for v in row] for row in c["dx"]])
            assert np.max(np.abs(dx - exp)) <= 1e-15, c["name"]
        else:
            dy = np.array([[float.fromhex(v) for v in row] for row in c["dy"]], dtype=np.float32)
            r = np.array([float.fromhex(v) for v in c["rstd"]], dtype=np.float32)
            dx, dw = orc.rmsnorm_backward(x, w, dy, r)
            exp_dx = np.array([[float(v) for v in row] for row in c["dx"]])
            exp_dw = np.array([float(v) for v in c["dw"]])
            assert np.max(np.abs(dx - exp_dx)) <= 1e-14 * np.max(np.abs(exp_dx)), c["name"]
            assert np.max(np.abs(dw - exp_dw)) <= 1e-14 * np.max(np.abs(exp_dw)), c["name"]
