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


class Stats:
    """Accuracy of one configuration against the oracle, over the elements checked:
    the largest relative error |g - r| / |r| (elements with |r| >= 2^-126), the largest
    error in units of the output type's ulp at r (2^(floor(log2|r|) - 23) for fp32,
    - 7 for bf16), and for bf16 outputs the fraction of elements that also meet the
    rounding bound |g - r| <= 2^-8 |r|.  Gradient outputs report the largest error as
    a fraction of their bound instead of a relative error."""

    def __init__(self, dtype: str, kind: str = "value"):
        self.dtype, self.kind = dtype, kind
        self.n = 0
        self.max_rel = 0.0
        self.max_ulp = 0.0
        self.max_bound = 0.0
        self.within = 0

    def add(self, n, max_rel=0.0, max_ulp=0.0, max_bound=0.0, within=0):
        self.n += int(n)
        self.max_rel = max(self.max_rel, float(max_rel))
        self.max_ulp = max(self.max_ulp, float(max_ulp))
        self.max_bound = max(self.max_bound, float(max_bound))
        self.within += int(within)
        return self

    def as_dict(self) -> dict:
        d = {"dtype": self.dtype, "kind": self.kind, "elements": self.n,
             "max_ulp": round(self.max_ulp, 4)}
        if self.kind == "value":
            d["max_rel_err"] = float(f"{self.max_rel:.4g}")
        else:
            d["max_err_over_bound"] = round(self.max_bound, 4)
        if self.dtype == "bf16" and self.kind == "value":
            d["frac_within_2^-8"] = round(self.within / max(1, self.n), 6)
        return d


def _ulp(r: np.ndarray, mant_bits: int) -> np.ndarray:
    ar = np.where(np.abs(r) < TINY, TINY, np.abs(r))
    return np.ldexp(1.0, np.floor(np.log2(ar)).astype(np.int64) - mant_bits)


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
    ulps = err / _ulp(r, 23) if err.size else np.zeros(1)
    return Stats("f32").add(g.size, rel.max() if rel.size else 0.0, ulps.max())


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
    if not g.size:
        return Stats("bf16")
    err = np.abs(g - r)
    rel = err[~tiny] / np.abs(r[~tiny]) if (~tiny).any() else np.zeros(1)
    within = np.count_nonzero(np.where(tiny, True, err <= np.ldexp(np.abs(r), -8)))
    return Stats("bf16").add(g.size, rel.max(), (err / np.where(tiny, 1.0, ulp)).max(),
                             within=within)


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
    if not g.size:
        return Stats(dtype, "gradient")
    ulps = err / _ulp(r, 23 if dtype == "f32" else 7)
    return Stats(dtype, "gradient").add(g.size, max_ulp=ulps.max(),
                                         max_bound=(err / np.maximum(bound, TINY)).max())


def check_rows_device(got, ref, dtype: str, stats: Stats, what=""):
    """Element-wise acceptance of a block of rows on the device: `got` a torch tensor
    of the output type (fp32 or bf16), `ref` the oracle's float64 values for the same
    rows (numpy, or a tensor already on the device).  Same bounds as check_f32 / check_bf16; adds to `stats`."""
    import torch

    r = (ref.double() if torch.is_tensor(ref)
         else torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float64)).to(got.device))
    g = got.double()
    assert g.shape == r.shape, (what, tuple(g.shape), tuple(r.shape))
    nan_r = torch.isnan(r)
    assert bool((torch.isnan(g) == nan_r).all()), f"{what}: NaN pattern differs"
    g = torch.where(nan_r, torch.zeros_like(g), g)
    r = torch.where(nan_r, torch.zeros_like(r), r)
    ar = r.abs()
    tiny = ar < TINY
    mant = 23 if dtype == "f32" else 7
    ulp = torch.ldexp(torch.ones_like(r),
                      torch.floor(torch.log2(ar.clamp_min(TINY))).to(torch.int32) - mant)
    err = (g - r).abs()
    tol = RTOL_F32 * ar if dtype == "f32" else ulp
    ok = torch.where(tiny, g.abs() < TINY, err <= tol) | nan_r
    if not bool(ok.all()):
        bad = torch.nonzero(~ok)[0].tolist()
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.numel()} outside the bound; "
                             f"first at {bad}: got {float(g[tuple(bad)])!r} "
                             f"ref {float(r[tuple(bad)])!r}")
    keep = ~tiny & ~nan_r
    rel = torch.where(keep, err / ar.clamp_min(TINY), torch.zeros_like(err))
    within = int((torch.where(keep, err <= ar * 2.0 ** -8, torch.ones_like(keep))
                  & ~nan_r).sum()) if dtype == "bf16" else 0
    return stats.add(int((~nan_r).sum()), float(rel.max()), float((err / ulp).max()),
                     within=within)
