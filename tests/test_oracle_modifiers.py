"""Pins for the score modifiers of the oracle (ALiBi slopes and softcap), on the CPU.

* a pure-Python brute force written from the definition (clamp the scaled
  score, subtract slope * distance, then mask), over every mask mode, GQA,
  Nq != Nk and per-batch slopes;
* closed forms: with zero queries and a causal mask, ALiBi weights are a
  geometric series; with a tiny softcap every visible logit saturates, so the
  output is the mean of the visible values and dQ = dK = 0;
* no-ops: slope 0 and a softcap far above every score change nothing;
* central finite differences of the loss pin the gradients with both modifiers;
* planted mistakes in copies of the oracle (sign, missing |.|, alignment,
  one-sided clamp, missing gradient gate, slopes not per batch entry) must each
  fail a compact pin.
"""

import inspect
import math
import types

import numpy as np
import pytest

import oracle
from oracle import attention as A
from test_oracle import MASKS, _close

MOD_MASKS = MASKS[:6]


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def brute_force_mod(q, k, v, causal, window, scale, slopes, softcap):
    """Loops over (b, h, i, j); slopes is (B, Hq) or None; softcap 0 = off."""
    nb, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    grp = hq // hkv
    wl, wr = window
    o = np.zeros(q.shape)
    lse = np.zeros((nb, hq, nq))
    for b in range(nb):
        for h in range(hq):
            g = h // grp
            for i in range(nq):
                logits = []
                for j in range(nk):
                    behind = (i + nk - nq) - j
                    if causal and behind < 0:
                        continue
                    if wl >= 0 and behind > wl:
                        continue
                    if wr >= 0 and -behind > wr:
                        continue
                    x = scale * sum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(d))
                    if softcap > 0:
                        x = max(-softcap, min(softcap, x))
                    if slopes is not None:
                        x -= float(slopes[b][h]) * abs(behind)
                    logits.append((j, x))
                if not logits:
                    lse[b, h, i] = -math.inf
                    continue
                den = sum(math.exp(x) for _, x in logits)
                for c in range(d):
                    o[b, i, h, c] = sum(math.exp(x) * float(v[b, j, g, c]) for j, x in logits) / den
                lse[b, h, i] = math.log(den)
    return o, lse


CASES = [(1, 5, 5, 2, 1, 3), (2, 4, 6, 4, 2, 2), (1, 6, 3, 2, 2, 3)]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("causal,window", MOD_MASKS)
@pytest.mark.parametrize("softcap", [0.0, 0.7])
def test_modifiers_match_brute_force(case, causal, window, softcap):
    nb, nq, nk, hq, hkv, d = case
    rng = np.random.default_rng(hash((case, causal, window, softcap)) % (2**32))
    q, k, v = _rand((nb, nq, hq, d), rng, 1.5), _rand((nb, nk, hkv, d), rng, 1.5), _rand((nb, nk, hkv, d), rng)
    slopes = rng.uniform(0.05, 1.0, (nb, hq))
    o, lse = oracle.attention_fwd(q, k, v, causal=causal, window=window, scale=0.8, alibi_slopes=slopes,
                                  softcap=softcap)
    ob, lb = brute_force_mod(q, k, v, causal, window, 0.8, slopes, softcap)
    assert _close(o, ob) and _close(lse, lb)
    # One slope vector for every batch entry.
    o1, l1 = oracle.attention_fwd(q, k, v, causal=causal, window=window, scale=0.8, alibi_slopes=slopes[0],
                                  softcap=softcap)
    ob1, lb1 = brute_force_mod(q, k, v, causal, window, 0.8, np.broadcast_to(slopes[0], slopes.shape), softcap)
    assert _close(o1, ob1) and _close(l1, lb1)


def test_alibi_with_zero_queries_is_a_geometric_series():
    # x = 0 everywhere: row i of a causal mask weighs key j by r^(i-j), r = e^-slope.
    rng = np.random.default_rng(1)
    n, d, slope = 7, 3, 0.4
    q = np.zeros((1, n, 1, d))
    k, v = _rand((1, n, 1, d), rng), _rand((1, n, 1, d), rng)
    o, lse = oracle.attention_fwd(q, k, v, causal=True, alibi_slopes=[slope])
    r = math.exp(-slope)
    for i in range(n):
        w = np.array([r ** (i - j) for j in range(i + 1)])
        assert np.allclose(o[0, i, 0], (w[:, None] * v[0, :i + 1, 0]).sum(0) / w.sum(), rtol=1e-13, atol=1e-13)
        assert math.isclose(lse[0, 0, i], math.log((1 - r ** (i + 1)) / (1 - r)), rel_tol=1e-13)


def test_tiny_softcap_saturates_every_logit():
    # All scores >= 0.5 and softcap 0.01: every visible logit is 0.01, so the
    # output is the mean of the visible values, LSE = 0.01 + ln(#visible), and
    # the clamp stops every gradient through the scores.
    rng = np.random.default_rng(2)
    n, d = 6, 4
    q = np.abs(_rand((1, n, 2, d), rng)) + 0.5
    k = np.abs(_rand((1, n, 1, d), rng)) + 0.5
    v, do = _rand((1, n, 1, d), rng), _rand((1, n, 2, d), rng)
    o, lse = oracle.attention_fwd(q, k, v, causal=True, scale=0.5, softcap=0.01)
    for i in range(n):
        assert np.allclose(o[0, i, :], v[0, :i + 1, 0].mean(0)[None, :], rtol=1e-13, atol=1e-13)
        assert np.allclose(lse[0, :, i], 0.01 + math.log(i + 1), rtol=1e-13)
    dq, dk, dv = oracle.attention_bwd(do, q, k, v, causal=True, scale=0.5, softcap=0.01)
    assert not np.any(dq) and not np.any(dk)
    _, _, dv0 = oracle.attention_bwd(do, np.zeros_like(q), k, v, causal=True, scale=0.5)
    assert np.allclose(dv, dv0, rtol=1e-13, atol=1e-13)  # uniform P either way


def test_neutral_modifiers_change_nothing():
    rng = np.random.default_rng(3)
    q, k, v, do = (_rand(s, rng) for s in ((2, 5, 4, 3), (2, 7, 2, 3), (2, 7, 2, 3), (2, 5, 4, 3)))
    o, lse = oracle.attention_fwd(q, k, v, causal=True)
    o2, lse2 = oracle.attention_fwd(q, k, v, causal=True, alibi_slopes=np.zeros(4), softcap=1e9)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    g = oracle.attention_bwd(do, q, k, v, causal=True)
    g2 = oracle.attention_bwd(do, q, k, v, causal=True, alibi_slopes=np.zeros(4), softcap=1e9)
    for x, y in zip(g, g2):
        assert np.array_equal(x, y)


def _fd_error(m, q, k, v, do, causal, window, scale, slopes, softcap, h=1e-6):
    grads = m.attention_bwd(do, q, k, v, causal=causal, window=window, scale=scale, alibi_slopes=slopes,
                            softcap=softcap)
    worst = 0.0
    for idx, x in enumerate((q, k, v)):
        for pos in np.ndindex(x.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[idx][pos] += h
            lp = np.sum(m.attention_fwd(*args, causal=causal, window=window, scale=scale, alibi_slopes=slopes,
                                        softcap=softcap)[0] * do)
            args[idx][pos] -= 2 * h
            lm = np.sum(m.attention_fwd(*args, causal=causal, window=window, scale=scale, alibi_slopes=slopes,
                                        softcap=softcap)[0] * do)
            worst = max(worst, abs((lp - lm) / (2 * h) - grads[idx][pos]) / max(1.0, abs(grads[idx][pos])))
    return worst


@pytest.mark.parametrize("causal,window", MOD_MASKS)
def test_gradients_match_finite_differences(causal, window):
    rng = np.random.default_rng(hash((causal, window, "mod")) % (2**32))
    q, k, v = _rand((1, 4, 2, 3), rng, 1.5), _rand((1, 5, 1, 3), rng, 1.5), _rand((1, 5, 1, 3), rng)
    do = _rand((1, 4, 2, 3), rng)
    # softcap 0.6 clamps part of the scores; the random scores are away from
    # +-0.6 by far more than the finite-difference step.
    assert _fd_error(A, q, k, v, do, causal, window, 0.9, np.array([[0.3, 0.8]]), 0.6) < 1e-7


# --------------------------------------------------------------------------
# Planted mistakes.
# --------------------------------------------------------------------------
MUTATIONS = [
    ("bias sign flipped", "out = out - slope * np.abs(aligned[:, None] - j[None, :])",
     "out = out + slope * np.abs(aligned[:, None] - j[None, :])"),
    ("distance without |.|", "out = out - slope * np.abs(aligned[:, None] - j[None, :])",
     "out = out - slope * (aligned[:, None] - j[None, :])"),
    ("bias aligned top-left", "aligned = np.asarray(rows, dtype=np.int64) - seqlen_q + seqlen_k",
     "aligned = np.asarray(rows, dtype=np.int64)"),
    ("one-sided clamp", "out = np.clip(x, -softcap, softcap)", "out = np.clip(x, None, softcap)"),
    ("clamp gate dropped", "ds = ds * gate", "ds = ds"),
    ("slopes not per batch entry", "return float(a[h] if a.ndim == 1 else a[b, h])",
     "return float(a[h] if a.ndim == 1 else a[0, h])"),
]


def _mutant(old, new):
    src = inspect.getsource(A)
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mod_mutant")
    exec(compile(src.replace(old, new), "oracle_mod_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(m):
    rng = np.random.default_rng(11)
    nb, nq, nk, hq, hkv, d = 2, 4, 5, 2, 1, 2
    q, k, v = _rand((nb, nq, hq, d), rng, 1.5), _rand((nb, nk, hkv, d), rng, 1.5), _rand((nb, nk, hkv, d), rng)
    do = _rand((nb, nq, hq, d), rng)
    slopes = rng.uniform(0.1, 1.0, (nb, hq))
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (False, (1, 1))]:
        o, lse = m.attention_fwd(q, k, v, causal=causal, window=window, scale=0.8, alibi_slopes=slopes, softcap=0.9)
        ob, lb = brute_force_mod(q, k, v, causal, window, 0.8, slopes, 0.9)
        if not (_close(o, ob) and _close(lse, lb)):
            return False
        if _fd_error(m, q, k, v, do, causal, window, 0.8, slopes, 0.9) > 1e-7:
            return False
    return True


def test_unmutated_copy_passes_the_compact_pins():
    assert _pins_pass(_mutant("import math", "import math"))


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    try:
        ok = _pins_pass(_mutant(old, new))
    except (ValueError, IndexError, FloatingPointError):
        ok = False
    assert not ok, f"planted mistake '{name}' was not caught by the pins"
