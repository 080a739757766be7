"""Comparison rule of the GPU results against the float64 oracle.

The tolerances are max-abs errors (fp32 1e-5, fp16 2e-3, bf16 1.6e-2 for O and
LSE; twice those for dQ/dK/dV).  An fp16/bf16 output cannot be closer to the
exact value than the nearest representable number of its type: at |x| in [8, 16)
a bf16 half-ulp is already 1/32 = 0.031, about the whole gradient bound.  So each
element is held to one of two bounds, chosen by the output type's spacing at
the exact value:

* raw: |gpu - ref| <= tol wherever the type's half-ulp at |ref| is at most
  tol / 2, i.e. wherever a correctly rounded output leaves at least half of
  the bound to the kernel (bf16 and fp16: |ref| < 4 for O, |ref| < 8 for the
  gradients; fp32: everywhere the tests reach);
* excess: above that band, |gpu - ref| - dist(ref, nearest value of the type)
  <= tol -- the error the kernel adds beyond the unavoidable output rounding.
"""

import numpy as np

MANTISSA_BITS = {"fp32": 23, "fp16": 10, "bf16": 7}
MIN_NORMAL_EXP = {"fp32": -126, "fp16": -14, "bf16": -126}


def _bf16_candidates(x):
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32) & np.uint32(0xFFFF0000)
    cands = []
    for delta in (0, 0x10000, -0x10000):
        b = (bits.astype(np.int64) + delta).clip(0, 0xFFFFFFFF).astype(np.uint32)
        cands.append(b.view(np.float32).astype(np.float64))
    return cands


def representation_distance(ref, dtype_name):
    """Distance from each float64 value to the nearest value of the output type."""
    ref = np.asarray(ref, dtype=np.float64)
    if dtype_name == "fp32":
        f = ref.astype(np.float32)
        cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    elif dtype_name == "fp16":
        f = ref.astype(np.float16)
        cands = [f, np.nextafter(f, np.float16(np.inf)), np.nextafter(f, np.float16(-np.inf))]
    elif dtype_name == "bf16":
        cands = _bf16_candidates(ref)
    else:
        raise ValueError(dtype_name)
    with np.errstate(invalid="ignore"):
        d = np.min([np.abs(ref - np.asarray(c, dtype=np.float64)) for c in cands], axis=0)
    return np.where(np.isfinite(d), d, 0.0)


def half_ulp(ref, dtype_name):
    """Half the spacing of the output type's values at |ref| (for |ref| on a power
    of two, the spacing above it)."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, MIN_NORMAL_EXP[dtype_name]), MIN_NORMAL_EXP[dtype_name])
    return np.ldexp(0.5, (e - MANTISSA_BITS[dtype_name]).astype(np.int64))


def raw_band_limit(dtype_name, tol):
    """Smallest |x| at which the type's half-ulp exceeds tol / 2: the raw bound
    holds for |ref| below it (inf if it holds at every finite magnitude below 2^100)."""
    for e in range(-30, 100):
        if half_ulp(np.array([2.0 ** e]), dtype_name)[0] > tol / 2:
            return 2.0 ** e
    return np.inf


def compare(got, ref, dtype_name, tol):
    """Statistics of one output against the oracle:
    raw       max |gpu - ref| over all finite entries (the literal max-abs error),
    raw_ref   |ref| at that worst element,
    raw_band  max |gpu - ref| where the raw bound applies,
    excess    max error beyond the output rounding where it does not (0 if none),
    band      |ref| below which the raw bound applies.
    Raises AssertionError on a different -inf pattern or non-finite GPU values."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), "-inf pattern differs"
    fin = ~inf_ref
    band = raw_band_limit(dtype_name, tol)
    info = dict(raw=0.0, raw_ref=0.0, raw_band=0.0, excess=0.0, band=band)
    if not fin.any():
        return info
    g, r = got[fin], ref[fin]
    assert np.all(np.isfinite(g)), "non-finite values in the GPU result"
    err = np.abs(g - r)
    w = int(np.argmax(err))
    info["raw"] = float(err[w])
    info["raw_ref"] = float(abs(r[w]))
    in_band = half_ulp(r, dtype_name) <= tol / 2
    if in_band.any():
        info["raw_band"] = float(err[in_band].max())
    if (~in_band).any():
        excess = err[~in_band] - representation_distance(r[~in_band], dtype_name)
        info["excess"] = float(max(excess.max(), 0.0))
    return info


def within(got, ref, dtype_name, tol):
    info = compare(got, ref, dtype_name, tol)
    return (info["raw_band"] <= tol and info["excess"] <= tol), info


def describe(info, tol):
    """One line: the literal max-abs error and where it sits, and the two bounds."""
    return (f"max-abs {info['raw']:.3e} at |ref| {info['raw_ref']:.3g}; raw bound (|ref| < {info['band']:g}) "
            f"{info['raw_band']:.3e}, excess above it {info['excess']:.3e}; tol {tol:.1e}")
