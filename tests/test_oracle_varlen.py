"""Pins for the packed variable-length oracle (oracle/varlen.py), on the CPU.

* equal lengths: the packed result is the fixed-length batch reshaped;
* unequal lengths: every sequence equals the pure-Python brute force of
  test_oracle.py run on that sequence alone (its own alignment of queries to
  keys), and the LSE lands at [head, packed row];
* finite differences of the packed loss pin the gradients;
* reordering the sequences reorders the results; empty sequences give
  -inf LSE and zero gradients; rows outside every sequence stay zero.
Planted mistakes in copies of the oracle must each fail a compact pin.
"""

import inspect
import types

import numpy as np
import pytest

import oracle
from oracle import varlen as VL
from test_oracle import _close, brute_force

MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (1, 0)), (True, (2, -1)), (False, (0, 2))]


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _packed(lens_q, lens_k, hq, hkv, d, rng, extra_q=0, extra_k=0):
    tq, tk = sum(lens_q) + extra_q, sum(lens_k) + extra_k
    q, k, v = _rand((tq, hq, d), rng), _rand((tk, hkv, d), rng), _rand((tk, hkv, d), rng)
    do = _rand((tq, hq, d), rng)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    return q, k, v, do, cu_q, cu_k


@pytest.mark.parametrize("causal,window", MASKS)
def test_equal_lengths_equal_the_fixed_length_batch(causal, window):
    rng = np.random.default_rng(1)
    b, n, hq, hkv, d = 3, 7, 4, 2, 5
    q, k, v, do, cu_q, cu_k = _packed([n] * b, [n] * b, hq, hkv, d, rng)
    o, lse = oracle.attention_fwd_varlen(q, k, v, cu_q, cu_k, causal=causal, window=window, scale=0.6)
    ob, lb = oracle.attention_fwd(q.reshape(b, n, hq, d), k.reshape(b, n, hkv, d), v.reshape(b, n, hkv, d),
                                  causal=causal, window=window, scale=0.6)
    assert _close(o, ob.reshape(b * n, hq, d))
    assert _close(lse, lb.transpose(1, 0, 2).reshape(hq, b * n))
    g = oracle.attention_bwd_varlen(do, q, k, v, cu_q, cu_k, causal=causal, window=window, scale=0.6)
    gb = oracle.attention_bwd(do.reshape(b, n, hq, d), q.reshape(b, n, hq, d), k.reshape(b, n, hkv, d),
                              v.reshape(b, n, hkv, d), causal=causal, window=window, scale=0.6)
    for x, y in zip(g, gb):
        assert _close(x, y.reshape(x.shape))


@pytest.mark.parametrize("causal,window", MASKS)
def test_each_sequence_matches_brute_force(causal, window):
    rng = np.random.default_rng(2)
    lens_q, lens_k = [3, 1, 5, 0, 4], [4, 6, 2, 3, 0]
    hq, hkv, d = 2, 1, 3
    q, k, v, _, cu_q, cu_k = _packed(lens_q, lens_k, hq, hkv, d, rng)
    o, lse = oracle.attention_fwd_varlen(q, k, v, cu_q, cu_k, causal=causal, window=window, scale=0.8)
    for b in range(len(lens_q)):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        ob, lb = brute_force(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], causal, window, 0.8)
        assert _close(o[q0:q1], ob[0]) and _close(lse[:, q0:q1], lb[0]), b


def test_gradients_match_finite_differences():
    rng = np.random.default_rng(3)
    q, k, v, do, cu_q, cu_k = _packed([2, 3], [3, 2], 2, 1, 2, rng)
    grads = oracle.attention_bwd_varlen(do, q, k, v, cu_q, cu_k, causal=True, scale=0.7)
    h = 1e-6
    for idx, x in enumerate((q, k, v)):
        for pos in np.ndindex(x.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[idx][pos] += h
            lp = np.sum(oracle.attention_fwd_varlen(*args, cu_q, cu_k, causal=True, scale=0.7)[0] * do)
            args[idx][pos] -= 2 * h
            lm = np.sum(oracle.attention_fwd_varlen(*args, cu_q, cu_k, causal=True, scale=0.7)[0] * do)
            assert abs((lp - lm) / (2 * h) - grads[idx][pos]) < 1e-7


def test_reordering_sequences_reorders_results():
    rng = np.random.default_rng(4)
    lens_q, lens_k = [2, 4, 3], [5, 1, 3]
    q, k, v, do, cu_q, cu_k = _packed(lens_q, lens_k, 2, 2, 3, rng)
    o, lse = oracle.attention_fwd_varlen(q, k, v, cu_q, cu_k, causal=True)
    perm = [2, 0, 1]
    qs = [q[cu_q[b]:cu_q[b + 1]] for b in perm]
    ks = [k[cu_k[b]:cu_k[b + 1]] for b in perm]
    vs = [v[cu_k[b]:cu_k[b + 1]] for b in perm]
    cq = np.concatenate([[0], np.cumsum([lens_q[b] for b in perm])])
    ck = np.concatenate([[0], np.cumsum([lens_k[b] for b in perm])])
    o2, lse2 = oracle.attention_fwd_varlen(np.concatenate(qs), np.concatenate(ks), np.concatenate(vs), cq, ck,
                                           causal=True)
    for j, b in enumerate(perm):
        assert np.array_equal(o2[cq[j]:cq[j + 1]], o[cu_q[b]:cu_q[b + 1]])
        assert np.array_equal(lse2[:, cq[j]:cq[j + 1]], lse[:, cu_q[b]:cu_q[b + 1]])


def test_empty_sequences_and_uncovered_rows():
    rng = np.random.default_rng(5)
    # sequence 1 has queries but no keys, sequence 2 keys but no queries; two
    # packed rows of q and k lie past the last sequence.
    q, k, v, do, cu_q, cu_k = _packed([2, 3, 0], [2, 0, 4], 2, 1, 3, rng, extra_q=2, extra_k=2)
    o, lse = oracle.attention_fwd_varlen(q, k, v, cu_q, cu_k)
    assert np.isneginf(lse[:, 2:5]).all() and not np.any(o[2:5])
    assert not np.any(o[5:]) and not np.any(lse[:, 5:])
    dq, dk, dv = oracle.attention_bwd_varlen(do, q, k, v, cu_q, cu_k)
    assert not np.any(dq[2:]) and not np.any(dk[2:]) and not np.any(dv[2:])
    assert np.any(dk[:2])


def test_invalid_offsets_are_rejected():
    q = np.zeros((4, 1, 2))
    for cq in ([1, 4], [0, 5], [0, 3, 2]):
        with pytest.raises(ValueError):
            oracle.attention_fwd_varlen(q, q, q, cq, [0, 4] if len(cq) == 2 else [0, 2, 4])


# --------------------------------------------------------------------------
# Planted mistakes.
# --------------------------------------------------------------------------
MUTATIONS = [
    ("sequence end off by one", "(int(cu_q[b]), int(cu_q[b + 1]),", "(int(cu_q[b]), int(cu_q[b + 1]) - 1,"),
    ("key range of the next sequence", "int(cu_k[b]), int(cu_k[b + 1]))", "int(cu_k[b]), int(cu_k[-1]))"),
    ("LSE rows not per sequence", "lse[:, q0:q1] = lb[0]", "lse[:, :q1 - q0] = lb[0]"),
    ("dK from the first sequence only", "dk[k0:k1], dv[k0:k1] = g[0][0], g[1][0], g[2][0]",
     "dk[0:k1 - k0], dv[k0:k1] = g[0][0], g[1][0], g[2][0]"),
]


def _mutant(old, new):
    src = inspect.getsource(VL)
    assert src.count(old) == 1, old
    src = src.replace(old, new).replace("from .attention import _as_f64, attention_bwd, attention_fwd", "")
    mod = types.ModuleType("varlen_mutant")
    from oracle import attention as A
    mod.__dict__.update(_as_f64=A._as_f64, attention_bwd=A.attention_bwd, attention_fwd=A.attention_fwd)
    exec(compile(src, "varlen_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(m):
    rng = np.random.default_rng(9)
    q, k, v, do, cu_q, cu_k = _packed([2, 3, 1], [3, 1, 2], 2, 1, 2, rng)
    for causal, window in MASKS[:3]:
        o, lse = m.attention_fwd_varlen(q, k, v, cu_q, cu_k, causal=causal, window=window, scale=0.8)
        for b in range(3):
            q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
            ob, lb = brute_force(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], causal, window, 0.8)
            if not (_close(o[q0:q1], ob[0]) and _close(lse[:, q0:q1], lb[0])):
                return False
        g = m.attention_bwd_varlen(do, q, k, v, cu_q, cu_k, causal=causal, window=window, scale=0.8)
        for b in range(3):
            q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
            gb = oracle.attention_bwd(do[None, q0:q1], q[None, q0:q1], k[None, k0:k1], v[None, k0:k1],
                                      causal=causal, window=window, scale=0.8)
            if not (_close(g[0][q0:q1], gb[0][0]) and _close(g[1][k0:k1], gb[1][0]) and
                    _close(g[2][k0:k1], gb[2][0])):
                return False
    return True


def test_unmutated_copy_passes_the_compact_pins():
    assert _pins_pass(_mutant("import numpy as np", "import numpy as np"))


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    try:
        ok = _pins_pass(_mutant(old, new))
    except (ValueError, IndexError):
        ok = False
    assert not ok, f"planted mistake '{name}' was not caught by the pins"
