"""Comparison rule of the GPU results against the float64 oracle.

The tolerances are max-abs errors (fp32 1e-5, fp16 2e-3, bf16 1.6e-2 for O and
LSE; twice those for dQ/dK/dV).  An fp16/bf16 output cannot be closer to the
exact value than the nearest representable number of its type: at |x| in [8, 16)
a bf16 half-ulp is already 0.031.  So two bounds are checked:

* excess: |gpu - ref| - dist(ref, nearest value of the output type) <= tol
  for every element -- the error the kernel adds beyond the output rounding;
* raw: |gpu - ref| <= tol for every element with |ref| < 4, where the output
  type's own rounding (at most 2^-7 for bf16) leaves most of the budget.
"""

import numpy as np

RAW_BOUND_MAGNITUDE = 4.0


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


def compare(got, ref, dtype_name, tol):
    """Returns (raw max-abs error, max excess error, raw max-abs error where |ref| < 4);
    raises AssertionError on a different -inf pattern or non-finite GPU values."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), "-inf pattern differs"
    fin = ~inf_ref
    if not fin.any():
        return 0.0, 0.0, 0.0
    g, r = got[fin], ref[fin]
    assert np.all(np.isfinite(g)), "non-finite values in the GPU result"
    err = np.abs(g - r)
    excess = err - representation_distance(r, dtype_name)
    small = np.abs(r) < RAW_BOUND_MAGNITUDE
    raw_small = float(err[small].max()) if small.any() else 0.0
    return float(err.max()), float(excess.max()), raw_small


def within(got, ref, dtype_name, tol):
    raw, excess, raw_small = compare(got, ref, dtype_name, tol)
    return (excess <= tol and raw_small <= tol), dict(raw=raw, excess=excess, raw_small=raw_small)
