"""Element-wise acceptance of GPU outputs against the oracle's float64 results.

fp32 outputs: |g - r| <= rtol * |r| with rtol = 1e-5; where |r| is below the
smallest normal fp32 (2^-126) the output passes if |g| is below it too.
bf16 outputs: g must be one of the two bf16 values that bracket r, i.e.
|g - r| <= ulp_bf16(r) = 2^(floor(log2|r|) - 7); the same subnormal rule applies.
NaN in the reference requires NaN in the output.
"""
import numpy as np

RTOL_F32 = 1e-5
TINY = 2.0 ** -126


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_f32(got, ref, what="", rtol=RTOL_F32):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    g, r = got[~nan_ref], ref[~nan_ref]
    tiny = np.abs(r) < TINY
    err = np.abs(g - r)
    ok = np.where(tiny, np.abs(g) < TINY, err <= rtol * np.abs(r))
    if not ok.all():
        i = np.flatnonzero(~ok)[0]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} of {ok.size} outside rel {rtol}; "
                             f"first at flat index {i}: got {g[i]!r} ref {r[i]!r}")
    rel = err[~tiny] / np.abs(r[~tiny]) if (~tiny).any() else np.zeros(1)
    return float(rel.max()) if rel.size else 0.0


def check_bf16(got_bits, ref, what=""):
    got = bf16_bits_to_f64(np.asarray(got_bits))
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    g, r = got[~nan_ref], ref[~nan_ref]
    tiny = np.abs(r) < TINY
    ar = np.where(tiny, 1.0, np.abs(r))
    ulp = np.ldexp(1.0, np.floor(np.log2(ar)).astype(np.int64) - 7)
    ok = np.where(tiny, np.abs(g) < TINY, np.abs(g - r) <= ulp)
    if not ok.all():
        i = np.flatnonzero(~ok)[0]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} of {ok.size} outside 1 bf16 ulp; "
                             f"first at flat index {i}: got {g[i]!r} ref {r[i]!r}")
    return float((np.abs(g - r) / np.where(tiny, 1.0, ulp)).max()) if g.size else 0.0
