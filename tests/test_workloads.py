"""CPU checks of the synthetic input recipes (no GPU, no oracle)."""

import numpy as np
import pytest
import torch

from exact_tiled_attention_07_amd.workloads import WORKLOADS, make_inputs, monotone_key_qkv, random_qkv

LAZY_RESCALE_LOG2 = 8.0  # growth of a row maximum (base 2) that the kernels absorb without rescaling


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tile,form", [(32, "steep"), (64, "steep"), (64, "mild")])
def test_monotone_keys_raise_every_tile_maximum(dtype, d, tile, form):
    # The adversaries of the rescale tests: for every query and every key tile
    # after the first, the tile's largest scaled score exceeds the largest of all
    # earlier tiles by more than the lazy-rescale margin, so a running maximum
    # moves (and the kernels rescale) on every tile.  32-key tiles are the
    # decode kernel's, 64-key tiles the forward's.
    if form == "steep":
        q, k, _, _ = monotone_key_qkv((1, 2048, 4, d), (1, 2048, 2, d), dtype, seed=3100 + d, rise_per_key=0.4)
    else:
        q, k, _, _ = monotone_key_qkv((1, 2048, 4, d), (1, 2048, 2, d), dtype, seed=3150 + d, rise_per_key=0.13,
                                      q_gain=4.0)
    qf = q.double().numpy()[0]
    kf = k.double().numpy()[0]
    for h in range(4):
        s = qf[:, h] @ kf[:, h // 2].T / np.sqrt(d) * np.log2(np.e)
        tmax = s.reshape(2048, 2048 // tile, tile).max(axis=2)
        rise = tmax[:, 1:] - np.maximum.accumulate(tmax, axis=1)[:, :-1]
        assert rise.min() > LAZY_RESCALE_LOG2, (h, rise.min())


def test_sigma_scales_inputs():
    q1, k1, v1, do1 = random_qkv((1, 64, 2, 64), (1, 64, 2, 64), "fp32", seed=9)
    q2, k2, v2, do2 = random_qkv((1, 64, 2, 64), (1, 64, 2, 64), "fp32", seed=9, sigma=2.0)
    assert torch.equal(q2, 2 * q1) and torch.equal(k2, 2 * k1) and torch.equal(v2, 2 * v1)
    assert torch.equal(do2, do1)  # dO keeps std 1


def test_workload_inputs_are_seeded_and_shaped():
    w = WORKLOADS["fp16_b2_h16_n512_d64_causal"]
    a = make_inputs(w)
    b = make_inputs(w)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert a[0].shape == w.q_shape and a[1].shape == w.kv_shape and a[0].dtype == torch.float16
