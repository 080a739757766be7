"""CPU checks of the rounding model that the stress tests compare against."""

import numpy as np
import pytest

import oracle
from exact_tiled_attention_07_amd.workloads import random_qkv
from rounding_model import policy_fwd, policy_grads, round_to


def _f64(*ts):
    return [t.double().numpy() for t in ts]


@pytest.mark.parametrize("mask", [dict(causal=True), dict(window=(5, 2))])
def test_model_without_rounding_is_the_oracle(mask):
    q, k, v, do = _f64(*random_qkv((2, 37, 4, 16), (2, 37, 2, 16), "fp32", seed=21))
    ref = oracle.attention_bwd(do, q, k, v, **mask)
    got = policy_grads(do, q, k, v, None, **mask)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype,u", [("bf16", 2.0 ** -8), ("fp16", 2.0 ** -11)])
def test_model_error_scales_with_the_unit_roundoff(dtype, u):
    # Each rounding moves a value by at most u relative, so the model's gradients
    # differ from the exact ones by a small multiple of u times their scale, and
    # by more than nothing.
    q, k, v, do = _f64(*random_qkv((1, 64, 2, 32), (1, 64, 1, 32), dtype, seed=22))
    ref = oracle.attention_bwd(do, q, k, v, causal=True)
    got = policy_grads(do, q, k, v, dtype, causal=True)
    for a, b in zip(got, ref):
        rel = np.abs(a - b).max() / np.abs(b).max()
        assert 0 < rel < 16 * u


def test_round_to_is_round_to_nearest_even():
    x = np.array([1.0 + 2.0 ** -9, 1.0 + 3 * 2.0 ** -9, -2.5])
    assert np.array_equal(round_to(x, "bf16"), [1.0, 1.0 + 2 * 2.0 ** -8, -2.5])


def test_forward_model_without_rounding_is_the_oracle():
    q, k, v, _ = _f64(*random_qkv((1, 45, 4, 16), (1, 45, 1, 16), "fp32", seed=23))
    o_ref, _ = oracle.attention_fwd(q, k, v, causal=True, window=(7, -1))
    assert np.allclose(policy_fwd(q, k, v, None, causal=True, window=(7, -1)), o_ref, rtol=1e-12, atol=1e-12)
