"""CPU checks of the comparison rule used by the GPU parity tests."""

import numpy as np

from compare import half_ulp, raw_band_limit, representation_distance, within


def _all_values(name):
    bits = np.arange(1 << 16, dtype=np.uint32)
    if name == "bf16":
        with np.errstate(invalid="ignore"):
            vals = (bits << 16).view(np.float32).astype(np.float64)
    else:
        vals = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    return np.unique(vals[np.isfinite(vals)])


def test_distance_matches_brute_force_over_every_value():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(2000) * s for s in (0.01, 1.0, 10.0, 300.0)])
    x = np.concatenate([x, [0.0, 1.0, -1.0, 1 + 2**-8, 9.203, -8.0 - 2**-6]])
    for name in ("bf16", "fp16"):
        grid = _all_values(name)
        idx = np.clip(np.searchsorted(grid, x), 1, len(grid) - 1)
        brute = np.minimum(np.abs(x - grid[idx - 1]), np.abs(x - grid[idx]))
        assert np.allclose(representation_distance(x, name), brute, rtol=0, atol=1e-18), name


def test_half_ulp_is_half_the_gap_to_the_next_value():
    # Brute force over every positive normal value of each 16-bit type: half the
    # distance to the next larger representable value.
    for name in ("bf16", "fp16"):
        grid = _all_values(name)
        tiny = 2.0 ** (-126 if name == "bf16" else -14)
        pos = grid[(grid >= tiny)]
        gaps = np.diff(pos) / 2
        assert np.array_equal(half_ulp(pos[:-1], name), gaps), name
        # values between two neighbours have the lower neighbour's spacing
        mid = (pos[:-1] + pos[1:]) / 2
        assert np.array_equal(half_ulp(-mid, name), gaps), name
    f = np.float32(3.0)
    assert half_ulp(np.array([3.0]), "fp32")[0] == (np.nextafter(f, np.float32(4)) - f) / 2


def test_raw_band_limits():
    # bf16/fp16: the raw bound covers |ref| < 4 at the O tolerances and < 8 at
    # the gradient tolerances (twice as large); fp32 far beyond any test value.
    assert raw_band_limit("bf16", 1.6e-2) == 4.0
    assert raw_band_limit("bf16", 3.2e-2) == 8.0
    assert raw_band_limit("fp16", 2e-3) == 4.0
    assert raw_band_limit("fp16", 4e-3) == 8.0
    assert raw_band_limit("fp32", 1e-5) == 128.0
    assert raw_band_limit("fp32", 1.6e-2) >= 2.0 ** 17  # LSE is fp32


def test_within_rule():
    ref = np.array([0.5, 9.2148, -3.9])
    # a correctly rounded bf16 output passes even where its own rounding exceeds tol
    got = np.array([0.5, 9.1875, -3.90625])
    ok, info = within(got, ref, "bf16", 0.016)
    assert ok and info["raw"] > 0.027 and info["excess"] < 1e-12 and info["raw_ref"] == 9.2148
    # an error beyond the rounding fails
    ok, _ = within(got + np.array([0.0, 0.125, 0.0]), ref, "bf16", 0.016)
    assert not ok
    # below |ref| = 4 the raw error alone must be within tol
    ok, _ = within(np.array([0.5, 9.1875, -3.88]), ref, "bf16", 0.016)
    assert not ok
    # -inf entries must match exactly
    ok, _ = within(np.array([-np.inf, 1.0]), np.array([-np.inf, 1.0]), "fp32", 1e-5)
    assert ok


def test_gradient_band_is_raw():
    # Gradient tolerance 0.032 in bf16: at |ref| in [4, 8) the raw bound applies
    # (a half-ulp there is 1/64, leaving half the bound to the kernel), so an error
    # of 0.03 passes only by the raw bound and 0.034 fails even though its excess
    # over the rounding is below the tolerance.
    ref = np.array([6.0 + 1 / 128])
    assert within(ref + 0.030, ref, "bf16", 0.032)[0]
    ok, info = within(ref + 0.034, ref, "bf16", 0.032)
    assert not ok and info["raw_band"] > 0.032
    # At |ref| in [8, 16) only the excess counts: 0.034 from the exact value is
    # within the bound when 0.0078 of it is the output's own rounding.
    ref = np.array([9.0 + 1 / 128])
    ok, info = within(np.array([9.0 + 1 / 128 + 0.034]), ref, "bf16", 0.032)
    assert ok and info["raw_band"] == 0.0
