"""Element-wise acceptance of GPU outputs against the oracle's float64 results.

fp32 outputs: |g - r| <= rtol * |r| with rtol = 1e-5; where |r| is below the
smallest normal fp32 (2^-126) the output passes if |g| is below it too.
bf16 outputs: g must be one of the two bf16 values that bracket r, i.e.
|g - r| <= ulp_bf16(r) = 2^(floor(log2|r|) - 7); the same subnormal rule applies.
NaN in the reference requires NaN in the output.

Gradient outputs (cross-entropy gradient, softmax and RMSNorm backward) are sums
of terms that can cancel (p - 1 at the label, dy - c, ...), so their bound is
relative to the size of the terms rather than to the result: with `scale` the
sum of the terms' magnitudes (given per element by the test),
fp32:  |g - r| <= 1e-5 * scale;  bf16:  |g - r| <= 1e-5 * scale + ulp_bf16(r)
(the fp32 result, then one rounding to bf16).  Where no cancellation happens
scale is |r| and the bound is the one above.
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


def check_grad(got, ref, scale, dtype, what="", rtol=RTOL_F32):
    """Gradient acceptance (see the module docstring); `got` is fp32 values or bf16
    bits, `scale` the per-element magnitude of the terms."""
    g = (np.asarray(got, dtype=np.float64) if dtype == "f32"
         else bf16_bits_to_f64(np.asarray(got)))
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.broadcast_to(np.asarray(scale, dtype=np.float64), ref.shape)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(g), nan_ref), f"{what}: NaN pattern differs"
    g, r, sc = g[~nan_ref], ref[~nan_ref], scale[~nan_ref]
    bound = rtol * sc + TINY
    if dtype != "f32":
        ar = np.where(np.abs(r) < TINY, 1.0, np.abs(r))
        bound = bound + np.where(np.abs(r) < TINY, TINY,
                                 np.ldexp(1.0, np.floor(np.log2(ar)).astype(np.int64) - 7))
    err = np.abs(g - r)
    ok = err <= bound
    if not ok.all():
        i = np.flatnonzero(~ok)[0]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} of {ok.size} outside the gradient "
                             f"bound; first at flat index {i}: got {g[i]!r} ref {r[i]!r} "
                             f"scale {sc[i]!r}")
    return float((err / np.maximum(bound, TINY)).max()) if g.size else 0.0
