import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle.default()


class _Overrides:
    """Accumulating test overrides of the library's planner and launcher (the
    rr_set_test_overrides entry point); cleared when the test ends."""

    def __init__(self):
        self.fields = {}

    def set(self, **kw):
        import memory_bound_row_softmax_amd as rr

        self.fields.update(kw)
        rr.set_test_overrides(**{k: v for k, v in self.fields.items() if v is not None})

    def clear(self):
        import memory_bound_row_softmax_amd as rr

        self.fields = {}
        rr.set_test_overrides()


@pytest.fixture
def overrides():
    o = _Overrides()
    try:
        yield o
    finally:
        o.clear()


def pytest_sessionfinish(session, exitstatus):
    """With RR_PARITY_LOG set, writes the accuracy lines the GPU tests recorded (one
    per configuration) as a markdown table next to the log (same name, .md)."""
    import json

    path = os.environ.get("RR_PARITY_LOG")
    if not path or not os.path.exists(path):
        return
    rows = [json.loads(l) for l in open(path) if l.strip()]
    out = os.path.splitext(path)[0] + ".md"
    with open(out, "w") as f:
        f.write("| configuration | output | elements checked | max rel. error | max ulp "
                "| max error / bound | bf16 within 2^-8 |r| |\n|---|---|---|---|---|---|---|\n")
        for d in rows:
            f.write(f"| {d['config']} | {d['dtype']} {d['kind']} | {d['elements']} | "
                    f"{d.get('max_rel_err', '')} | {d['max_ulp']} | "
                    f"{d.get('max_err_over_bound', '')} | {d.get('frac_within_2^-8', '')} |\n")
