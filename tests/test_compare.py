"""CPU checks of the comparison rule used by the GPU parity tests."""

import numpy as np

from compare import representation_distance, within


def _all_values(name):
    bits = np.arange(1 << 16, dtype=np.uint32)
    if name == "bf16":
        vals = (bits << 16).view(np.float32).astype(np.float64)
    else:
        vals = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    return np.sort(vals[np.isfinite(vals)])


def test_distance_matches_brute_force_over_every_value():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(2000) * s for s in (0.01, 1.0, 10.0, 300.0)])
    x = np.concatenate([x, [0.0, 1.0, -1.0, 1 + 2**-8, 9.203, -8.0 - 2**-6]])
    for name in ("bf16", "fp16"):
        grid = _all_values(name)
        idx = np.clip(np.searchsorted(grid, x), 1, len(grid) - 1)
        brute = np.minimum(np.abs(x - grid[idx - 1]), np.abs(x - grid[idx]))
        assert np.allclose(representation_distance(x, name), brute, rtol=0, atol=1e-18), name


def test_within_rule():
    ref = np.array([0.5, 9.2148, -3.9])
    # a correctly rounded bf16 output passes even where its own rounding exceeds tol
    got = np.array([0.5, 9.1875, -3.90625])
    ok, info = within(got, ref, "bf16", 0.016)
    assert ok and info["raw"] > 0.027 and info["excess"] < 1e-12
    # an error beyond the rounding fails
    ok, _ = within(got + np.array([0.0, 0.125, 0.0]), ref, "bf16", 0.016)
    assert not ok
    # below |ref| = 4 the raw error alone must be within tol
    ok, _ = within(np.array([0.5, 9.1875, -3.88]), ref, "bf16", 0.016)
    assert not ok
    # -inf entries must match exactly
    ok, _ = within(np.array([-np.inf, 1.0]), np.array([-np.inf, 1.0]), "fp32", 1e-5)
    assert ok
