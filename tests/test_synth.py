"""The shared input generator: determinism, row independence, distributions."""
import numpy as np
import pytest

import synth
from synth import workloads as W


def test_deterministic_and_seeded():
    a = synth.normal(8, 300)
    b = synth.normal(8, 300)
    c = synth.normal(8, 300, seed=synth.SEED + 1)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rows_regenerate_independently(dtype):
    full = synth.normal(64, 777, dtype=dtype)
    rows = [0, 3, 63, 17]
    assert np.array_equal(synth.normal(64, 777, dtype=dtype, rows=rows), full[rows])
    assert np.array_equal(synth.normal(10, 777, dtype=dtype, row0=20), full[20:30])
    # element (row, col) does not depend on M
    assert np.array_equal(synth.normal(2000, 777, dtype=dtype, nthreads=4)[:64], full)


def test_threading_does_not_change_values():
    a = synth.normal(512, 1024, nthreads=1)
    b = synth.normal(512, 1024, nthreads=7)
    assert np.array_equal(a, b)


def test_normal_moments():
    x = synth.normal(256, 4096, sigma=2.0).astype(np.float64)
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 2.0) < 0.01
    # tails of a Gaussian: P(|z| > 3) ~ 0.0027
    assert abs(np.mean(np.abs(x) > 6.0) - 0.0027) < 0.0005


def test_uniform_range_and_mean():
    u = synth.uniform(64, 4096, lo=0.5, hi=1.5).astype(np.float64)
    assert u.min() >= 0.5 and u.max() <= 1.5
    assert abs(u.mean() - 1.0) < 0.005


def test_bf16_is_rne_of_f32():
    f = synth.normal(16, 512)
    b = synth.normal(16, 512, dtype="bf16")
    assert np.array_equal(b, synth.f32_to_bf16(f))
    # decode and check the rounding is to the nearest bf16 value
    dec = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(dec))[1] - 8)
    assert np.all(np.abs(dec - f) <= ulp / 2 + 1e-30)


def test_f32_to_bf16_ties_and_specials():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.0, 0.0, np.inf, np.nan],
                    dtype=np.float32)
    out = synth.f32_to_bf16(vals)
    assert out[0] == 0x3F80
    assert out[1] == 0x3F80          # tie -> even (down)
    assert out[2] == 0x3F82          # tie -> even (up)
    assert out[3] == 0xC000
    assert out[4] == 0x0000
    assert out[5] == 0x7F80
    assert (out[6] & 0x7F80) == 0x7F80 and (out[6] & 0x7F) != 0


def test_spike_rate_and_value():
    x = W.x_rows(W.SOFTMAX_SPIKY, nrows=8)
    rate = np.mean(x == 20.0)
    assert 0.009 < rate < 0.011
    again = W.x_rows(W.SOFTMAX_SPIKY, rows=[5, 2])
    assert np.array_equal(again, x[[5, 2]])


def test_labels_in_range_and_uniform():
    lab = synth.labels(200000, 1000)
    assert lab.min() >= 0 and lab.max() < 1000
    counts = np.bincount(lab, minlength=1000)
    assert counts.min() > 100 and counts.max() < 320
    assert np.array_equal(synth.labels(200000, 1000, rows=[7, 199999]), lab[[7, 199999]])


def test_workload_table():
    names = [w.name for w in W.FIXED]
    assert names[1] == "rmsnorm_bf16_16384x4096"
    assert len(W.sweep()) == 3 * 2 * 3 * 6
    assert W.by_name("xent_f32_8192x131072").sigma == 2.0
