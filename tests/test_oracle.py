"""Pins for the float64 oracle, on the CPU.

Each check ties the oracle to something other than itself: a pure-Python brute
force written from the definition (no max subtraction, masks written as
distances), closed forms, invariants of softmax attention, central finite
differences of the loss, a hand-derived golden example, and a float64 library
cross-check (torch's scaled_dot_product_attention on the CPU).  The last group
plants mistakes in copies of the oracle and checks that the pins catch every one.
"""

import inspect
import json
import math
import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention as A

HERE = os.path.dirname(os.path.abspath(__file__))

# (causal, (window_left, window_right)) combinations used throughout.
MASKS = [
    (False, (-1, -1)), (True, (-1, -1)), (False, (0, 0)), (False, (1, 0)),
    (False, (2, 1)), (True, (2, -1)), (False, (-1, 1)), (True, (0, 3)),
]


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


# --------------------------------------------------------------------------
# Brute force: loops over every (b, h, i, j), math.exp without the max shift.
# --------------------------------------------------------------------------
def brute_force(q, k, v, causal, window, scale):
    nb, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    per_group = hq // hkv
    wl, wr = window
    o = np.zeros(q.shape)
    lse = np.zeros((nb, hq, nq))
    for b in range(nb):
        for g in range(hkv):
            for h in range(g * per_group, (g + 1) * per_group):
                for i in range(nq):
                    num = [0.0] * d
                    den = 0.0
                    for j in range(nk):
                        # how many positions key j lies behind query i, with the
                        # last query aligned to the last key
                        behind = (i + nk - nq) - j
                        if causal and behind < 0:
                            continue
                        if wl >= 0 and behind > wl:
                            continue
                        if wr >= 0 and -behind > wr:
                            continue
                        s = scale * sum(float(q[b, i, h, c]) * float(k[b, j, g, c]) for c in range(d))
                        e = math.exp(s)
                        den += e
                        for c in range(d):
                            num[c] += e * float(v[b, j, g, c])
                    if den == 0.0:
                        lse[b, h, i] = -math.inf
                    else:
                        o[b, i, h, :] = [x / den for x in num]
                        lse[b, h, i] = math.log(den)
    return o, lse


def _close(a, b, rtol=1e-12, atol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    same_inf = (np.isneginf(a) == np.isneginf(b)).all()
    fin = np.isfinite(b)
    return bool(same_inf and np.allclose(a[fin], b[fin], rtol=rtol, atol=atol))


BF_CASES = [
    # (batch, nq, nk, hq, hkv, d)
    (1, 5, 5, 1, 1, 3),
    (2, 6, 6, 4, 2, 4),
    (1, 4, 6, 4, 1, 2),   # Nq < Nk: bottom-right alignment
    (2, 6, 3, 2, 2, 3),   # Nq > Nk: leading rows may see nothing under masks
    (1, 1, 6, 4, 4, 4),   # single query against six keys
]


@pytest.mark.parametrize("case", BF_CASES)
@pytest.mark.parametrize("causal,window", MASKS)
def test_forward_matches_brute_force(case, causal, window):
    nb, nq, nk, hq, hkv, d = case
    rng = np.random.default_rng(hash((case, causal, window)) % (2**32))
    q = _rand((nb, nq, hq, d), rng)
    k = _rand((nb, nk, hkv, d), rng)
    v = _rand((nb, nk, hkv, d), rng)
    scale = 0.7
    o, lse = oracle.attention_fwd(q, k, v, causal=causal, window=window, scale=scale)
    o_bf, lse_bf = brute_force(q, k, v, causal, window, scale)
    assert _close(o, o_bf)
    assert _close(lse, lse_bf)


def test_forward_rows_matches_full():
    rng = np.random.default_rng(5)
    q, k, v = _rand((2, 40, 4, 8), rng), _rand((2, 40, 2, 8), rng), _rand((2, 40, 2, 8), rng)
    o, lse = oracle.attention_fwd(q, k, v, causal=True, window=(5, -1))
    rows = np.array([0, 3, 17, 39])
    orow, lrow = oracle.attention_fwd_rows(q, k, v, 1, 3, rows, causal=True, window=(5, -1))
    assert np.allclose(orow, o[1, rows, 3], rtol=1e-13, atol=1e-13)
    assert np.allclose(lrow, lse[1, 3, rows], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Closed forms.
# --------------------------------------------------------------------------
def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(1)
    n, w = 20, 3
    q = np.zeros((1, n, 2, 4))
    k, v = _rand((1, n, 2, 4), rng), _rand((1, n, 2, 4), rng)
    o, lse = oracle.attention_fwd(q, k, v, causal=True)
    o_w, lse_w = oracle.attention_fwd(q, k, v, causal=True, window=(w, 0))
    for i in range(n):
        for h in range(2):
            # causal: keys 0..i are visible
            assert np.allclose(o[0, i, h], v[0, : i + 1, h].mean(axis=0), atol=1e-14)
            assert abs(lse[0, h, i] - math.log(i + 1)) < 1e-14
            # sliding window (w, 0): keys max(0, i - w)..i are visible
            lo = max(0, i - w)
            assert np.allclose(o_w[0, i, h], v[0, lo: i + 1, h].mean(axis=0), atol=1e-14)
            assert abs(lse_w[0, h, i] - math.log(i + 1 - lo)) < 1e-14


def test_causal_row_zero_is_first_value():
    rng = np.random.default_rng(2)
    q, k, v = _rand((2, 9, 3, 5), rng), _rand((2, 9, 3, 5), rng), _rand((2, 9, 3, 5), rng)
    scale = 0.37
    o, lse = oracle.attention_fwd(q, k, v, causal=True, scale=scale)
    assert np.array_equal(o[:, 0], v[:, 0])
    assert np.allclose(lse[:, :, 0], scale * np.einsum("bhc,bhc->bh", q[:, 0], k[:, 0]), atol=1e-14)


def test_window_self_only_returns_values():
    rng = np.random.default_rng(3)
    q, k, v = _rand((1, 11, 4, 6), rng), _rand((1, 11, 2, 6), rng), _rand((1, 11, 2, 6), rng)
    scale = 0.5
    o, lse = oracle.attention_fwd(q, k, v, window=(0, 0), scale=scale)
    for h in range(4):
        g = h // 2
        assert np.array_equal(o[0, :, h], v[0, :, g])
        assert np.allclose(lse[0, h], scale * np.sum(q[0, :, h] * k[0, :, g], axis=1), atol=1e-14)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(4)
    q, k = _rand((1, 13, 2, 4), rng), _rand((1, 13, 2, 4), rng)
    c = np.array([1.5, -2.0, 0.25, 3.0])
    v = np.broadcast_to(c, (1, 13, 2, 4)).copy()
    for causal, window in MASKS[:5]:
        o, _ = oracle.attention_fwd(q, k, v, causal=causal, window=window)
        assert np.allclose(o, c, atol=1e-14)


def test_gqa_equals_mha_on_repeated_heads():
    rng = np.random.default_rng(6)
    q = _rand((2, 12, 8, 4), rng)
    k, v = _rand((2, 12, 2, 4), rng), _rand((2, 12, 2, 4), rng)
    do = _rand((2, 12, 8, 4), rng)
    k4, v4 = np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2)
    o, lse = oracle.attention_fwd(q, k, v, causal=True)
    o4, lse4 = oracle.attention_fwd(q, k4, v4, causal=True)
    assert np.allclose(o, o4, atol=1e-14) and np.allclose(lse, lse4, atol=1e-14)
    dq, dk, dv = oracle.attention_bwd(do, q, k, v, causal=True)
    dq4, dk4, dv4 = oracle.attention_bwd(do, q, k4, v4, causal=True)
    assert np.allclose(dq, dq4, atol=1e-13)
    # the group's K/V gradient is the sum of its repeated copies
    assert np.allclose(dk, dk4.reshape(2, 12, 2, 4, 4).sum(axis=3), atol=1e-13)
    assert np.allclose(dv, dv4.reshape(2, 12, 2, 4, 4).sum(axis=3), atol=1e-13)


def test_causal_is_right_window_zero_and_unbounded_window_is_none():
    rng = np.random.default_rng(7)
    q, k, v = _rand((1, 10, 2, 3), rng), _rand((1, 10, 2, 3), rng), _rand((1, 10, 2, 3), rng)
    a = oracle.attention_fwd(q, k, v, causal=True)
    b = oracle.attention_fwd(q, k, v, window=(-1, 0))
    c = oracle.attention_fwd(q, k, v, causal=True, window=(-1, 4))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    for x, y in zip(a, c):
        assert np.array_equal(x, y)
    d = oracle.attention_fwd(q, k, v)
    e = oracle.attention_fwd(q, k, v, window=(100, 100))
    for x, y in zip(d, e):
        assert np.array_equal(x, y)


def test_rows_without_visible_keys():
    rng = np.random.default_rng(8)
    # Nq > Nk with causal bottom-right alignment: the first Nq - Nk rows see nothing
    q, k, v = _rand((1, 7, 2, 3), rng), _rand((1, 4, 2, 3), rng), _rand((1, 4, 2, 3), rng)
    do = _rand((1, 7, 2, 3), rng)
    o, lse = oracle.attention_fwd(q, k, v, causal=True)
    assert np.all(o[0, :3] == 0.0) and np.all(np.isneginf(lse[0, :, :3]))
    assert np.all(np.isfinite(lse[0, :, 3:]))
    dq, dk, dv = oracle.attention_bwd(do, q, k, v, causal=True)
    assert np.all(dq[0, :3] == 0.0)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))


# --------------------------------------------------------------------------
# Invariants.
# --------------------------------------------------------------------------
def test_softmax_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(9)
    s = _rand((16, 23), rng, 3.0)
    vis = oracle.visible(16, 23, causal=True, window=(6, -1))
    p, lse = oracle.masked_softmax(s, vis)
    assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 1e-12)
    assert np.all(p[~vis] == 0.0)
    shift = _rand((16,), rng, 50.0)
    p2, lse2 = oracle.masked_softmax(s + shift[:, None], vis)
    assert np.allclose(p2, p, atol=1e-12)
    assert np.allclose(lse2, lse + shift, atol=1e-10)


def test_key_shift_moves_lse_not_output():
    # K -> K + 1 u^T adds scale * (q_i . u) to every score of row i.
    rng = np.random.default_rng(10)
    q, k, v = _rand((1, 9, 2, 4), rng), _rand((1, 9, 1, 4), rng), _rand((1, 9, 1, 4), rng)
    u = _rand((4,), rng)
    scale = 0.5
    o, lse = oracle.attention_fwd(q, k, v, causal=True, scale=scale)
    o2, lse2 = oracle.attention_fwd(q, k + u, v, causal=True, scale=scale)
    assert np.allclose(o2, o, atol=1e-12)
    assert np.allclose(lse2, lse + scale * np.einsum("bihc,c->bhi", q, u), atol=1e-12)


def test_permutations_and_linearity():
    rng = np.random.default_rng(11)
    q, k, v = _rand((1, 8, 2, 3), rng), _rand((1, 10, 2, 3), rng), _rand((1, 10, 2, 3), rng)
    v2 = _rand((1, 10, 2, 3), rng)
    o, lse = oracle.attention_fwd(q, k, v)
    pk = rng.permutation(10)
    o_k, lse_k = oracle.attention_fwd(q, k[:, pk], v[:, pk])
    assert np.allclose(o_k, o, atol=1e-13) and np.allclose(lse_k, lse, atol=1e-13)
    pq = rng.permutation(8)
    o_q, lse_q = oracle.attention_fwd(q[:, pq], k, v)
    assert np.allclose(o_q, o[:, pq], atol=1e-14) and np.allclose(lse_q, lse[:, :, pq], atol=1e-14)
    o_lin, _ = oracle.attention_fwd(q, k, v + 2.0 * v2)
    o_v2, _ = oracle.attention_fwd(q, k, v2)
    assert np.allclose(o_lin, o + 2.0 * o_v2, atol=1e-12)


# --------------------------------------------------------------------------
# Gradients: central finite differences of L = sum(O * dO).
# --------------------------------------------------------------------------
def fd_gradient_error(fwd, bwd, q, k, v, do, causal, window, scale, h=1e-6):
    grads = bwd(do, q, k, v, causal=causal, window=window, scale=scale)
    worst = 0.0
    for idx, x in enumerate((q, k, v)):
        for pos in np.ndindex(x.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[idx][pos] += h
            lp = np.sum(fwd(*args, causal=causal, window=window, scale=scale)[0] * do)
            args[idx][pos] -= 2 * h
            lm = np.sum(fwd(*args, causal=causal, window=window, scale=scale)[0] * do)
            fd = (lp - lm) / (2 * h)
            g = grads[idx][pos]
            worst = max(worst, abs(fd - g) / max(1.0, abs(g)))
    return worst


FD_CASES = [(1, 4, 4, 2, 1, 3), (2, 3, 3, 2, 2, 2), (1, 3, 5, 4, 2, 2), (1, 5, 3, 2, 1, 2)]


@pytest.mark.parametrize("case", FD_CASES)
@pytest.mark.parametrize("causal,window", MASKS)
def test_backward_matches_finite_differences(case, causal, window):
    nb, nq, nk, hq, hkv, d = case
    rng = np.random.default_rng(hash((case, causal, window, "fd")) % (2**32))
    q, k, v = _rand((nb, nq, hq, d), rng), _rand((nb, nk, hkv, d), rng), _rand((nb, nk, hkv, d), rng)
    do = _rand((nb, nq, hq, d), rng)
    err = fd_gradient_error(oracle.attention_fwd, oracle.attention_bwd, q, k, v, do, causal, window, 0.8)
    assert err <= 1e-7


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (3, -1))])
def test_gradient_identities(causal, window):
    rng = np.random.default_rng(12)
    q, k, v = _rand((2, 14, 4, 5), rng), _rand((2, 14, 2, 5), rng), _rand((2, 14, 2, 5), rng)
    do = _rand((2, 14, 4, 5), rng)
    dq, dk, dv = oracle.attention_bwd(do, q, k, v, causal=causal, window=window)
    # rows of dS sum to zero, so the key gradients sum to zero per K/V head
    assert np.allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # every row sees at least one key, so dV sums to the group's dO
    assert np.allclose(dv.sum(axis=1), do.reshape(2, 14, 2, 2, 5).sum(axis=(1, 3)), atol=1e-12)


# --------------------------------------------------------------------------
# Hand-derived golden example (tests/golden/hand_example_n2_d2.json).
# --------------------------------------------------------------------------
def _golden_value(x):
    if isinstance(x, list):
        return [_golden_value(y) for y in x]
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}},
                          {"ln3": math.log(3), "ln4": math.log(4), "ln7": math.log(7),
                           "ln8": math.log(8)}))
    return float(x)


def test_hand_derived_golden_example():
    with open(os.path.join(HERE, "golden", "hand_example_n2_d2.json")) as f:
        gold = json.load(f)
    inp = gold["inputs"]
    q, k, v, do = (np.array(_golden_value(inp[n]))[None] for n in ("q", "k", "v", "do"))
    for mode, causal in (("noncausal", False), ("causal", True)):
        exp = gold["expected"][mode]
        o, lse = oracle.attention_fwd(q, k, v, causal=causal, scale=inp["scale"])
        dq, dk, dv = oracle.attention_bwd(do, q, k, v, causal=causal, scale=inp["scale"])
        assert np.allclose(o, np.array(_golden_value(exp["o"]))[None], atol=1e-14)
        assert np.allclose(lse, np.array(_golden_value(exp["lse"]))[None], atol=1e-14)
        for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            assert np.allclose(got, np.array(_golden_value(exp[name]))[None], atol=1e-14), name


# --------------------------------------------------------------------------
# Library cross-check: torch SDPA on the CPU in float64 (never used by the oracle).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(4, 4), (4, 2), (6, 1)])
def test_matches_torch_sdpa_float64(causal, heads):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    hq, hkv = heads
    rng = np.random.default_rng(13)
    q, k, v = _rand((2, 37, hq, 16), rng), _rand((2, 37, hkv, 16), rng), _rand((2, 37, hkv, 16), rng)
    do = _rand((2, 37, hq, 16), rng)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.transpose(1, 2), tv.transpose(1, 2),
        is_causal=causal, scale=0.3, enable_gqa=(hq != hkv)).transpose(1, 2)
    (out * torch.tensor(do)).sum().backward()
    o, _ = oracle.attention_fwd(q, k, v, causal=causal, scale=0.3)
    dq, dk, dv = oracle.attention_bwd(do, q, k, v, causal=causal, scale=0.3)
    assert np.allclose(o, out.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Planted mistakes: each mutated copy of the oracle must fail some pin above.
# --------------------------------------------------------------------------
MUTATIONS = [
    ("exclusive causal bound", "vis &= j <= i\n", "vis &= j < i\n"),
    ("exclusive left window", "vis &= j >= i - wl", "vis &= j > i - wl"),
    ("right window ignored", "vis &= j <= i + wr", "vis &= j <= i + wr + 1"),
    ("top-left alignment", "[:, None] + (seqlen_k - seqlen_q)", "[:, None] + 0"),
    ("strided head map", "return h // (nheads_q // nheads_kv)", "return h % nheads_kv"),
    ("scale dropped", "return scale * (_as_f64(q_rows) @ _as_f64(k_head).T)",
     "return (_as_f64(q_rows) @ _as_f64(k_head).T)"),
    ("lse without the row max", "m_safe + np.log(", "np.log("),
    ("no normalisation", "p = e / denom[:, None]", "p = e"),
    ("D term dropped", "ds = p * (dp - dsum[:, None])", "ds = p * dp"),
    ("wrong sign in dS", "ds = p * (dp - dsum[:, None])", "ds = p * (dsum[:, None] - dp)"),
    ("dQ scale dropped", "dq[b, r0:r1, h, :] = scale * (ds @ kh)", "dq[b, r0:r1, h, :] = (ds @ kh)"),
    ("dK uses dO", "dk[b, :, g, :] += scale * (ds.T @ qr)", "dk[b, :, g, :] += scale * (ds.T @ dor)"),
    ("dV uses dS", "dv[b, :, g, :] += p.T @ dor", "dv[b, :, g, :] += ds.T @ dor"),
    ("dK overwritten per head", "dk[b, :, g, :] += scale", "dk[b, :, g, :] = scale"),
]


def _mutant(src_old, src_new):
    src = inspect.getsource(A)
    assert src.count(src_old) == 1, src_old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(src_old, src_new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(m):
    """Run a compact version of the pins above against module ``m``."""
    rng = np.random.default_rng(99)
    for case in [(1, 4, 4, 4, 2, 2), (1, 3, 5, 2, 1, 2), (1, 5, 3, 2, 2, 2)]:
        nb, nq, nk, hq, hkv, d = case
        q, k, v = _rand((nb, nq, hq, d), rng), _rand((nb, nk, hkv, d), rng), _rand((nb, nk, hkv, d), rng)
        do = _rand((nb, nq, hq, d), rng)
        for causal, window in MASKS:
            o, lse = m.attention_fwd(q, k, v, causal=causal, window=window, scale=0.8)
            o_bf, lse_bf = brute_force(q, k, v, causal, window, 0.8)
            if not (_close(o, o_bf) and _close(lse, lse_bf)):
                return False
            if fd_gradient_error(m.attention_fwd, m.attention_bwd, q, k, v, do, causal, window, 0.8) > 1e-7:
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
