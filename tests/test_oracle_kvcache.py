"""Pins for the KV-cache oracle (oracle/kvcache.py), on the CPU.

The decode oracle is tied to things other than itself:

* token-by-token decoding and chunked prefill reproduce the rows of one full
  causal (or windowed) attention over the whole sequence -- what incremental
  decoding exists to compute;
* a pure-Python brute force that builds each batch entry's key list as "the
  valid cache rows, then the new rows while capacity lasts" and loops over it;
* cache rows past the valid length (filled with NaN) never reach the result;
* batch entries are independent, and the in-place append moves exactly the
  rows the reading says it does.

Planted mistakes in copies of the oracle (append offset, key count, alignment)
must each fail one of the compact pins.
"""

import inspect
import math
import types

import numpy as np
import pytest

import oracle
from oracle import kvcache as KV


def _rand(shape, rng):
    return rng.standard_normal(shape)


def brute_decode(q, kc, vc, lens, kn, vn, causal, window, scale):
    """Loops over (b, h, i, key); keys are listed explicitly, old then new."""
    nb, nq, hq, d = q.shape
    cap, hkv = kc.shape[1], kc.shape[2]
    grp = hq // hkv
    wl, wr = window
    o = np.zeros(q.shape)
    lse = np.zeros((nb, hq, nq))
    for b in range(nb):
        length = min(max(int(lens[b]), 0), cap)
        keys = [(kc[b, j], vc[b, j]) for j in range(length)]
        if kn is not None:
            for i in range(nq):
                if len(keys) < cap:
                    keys.append((kn[b, i], vn[b, i]))
        nk = len(keys)
        for h in range(hq):
            g = h // grp
            for i in range(nq):
                num = [0.0] * d
                den = 0.0
                for j, (kr, vr) in enumerate(keys):
                    behind = (nk - nq + i) - j     # last query sits on the last key
                    if causal and behind < 0:
                        continue
                    if wl >= 0 and behind > wl:
                        continue
                    if wr >= 0 and -behind > wr:
                        continue
                    s = scale * sum(float(q[b, i, h, c]) * float(kr[g, c]) for c in range(d))
                    e = math.exp(s)
                    den += e
                    for c in range(d):
                        num[c] += e * float(vr[g, c])
                if den == 0.0:
                    lse[b, h, i] = -math.inf
                else:
                    o[b, i, h] = [x / den for x in num]
                    lse[b, h, i] = math.log(den)
    return o, lse


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    if not np.array_equal(np.isneginf(a), np.isneginf(b)):
        return False
    fin = np.isfinite(b)
    return bool(np.allclose(a[fin], b[fin], rtol=tol, atol=tol))


MASKS = [(False, (-1, -1)), (True, (-1, -1)), (True, (2, -1)), (False, (1, 1)), (False, (0, 0))]


@pytest.mark.parametrize("causal,window", MASKS)
def test_token_by_token_decode_equals_full_attention(causal, window):
    rng = np.random.default_rng(1)
    n, hq, hkv, d, cap = 9, 4, 2, 5, 12
    q, k, v = _rand((2, n, hq, d), rng), _rand((2, n, hkv, d), rng), _rand((2, n, hkv, d), rng)
    o_full, lse_full = oracle.attention_fwd(q, k, v, causal=causal, window=window, scale=0.6)
    kc = np.full((2, cap, hkv, d), np.nan)
    vc = np.full((2, cap, hkv, d), np.nan)
    lens = np.zeros(2, dtype=np.int64)
    for t in range(n):
        o, lse, kc, vc = oracle.kvcache_fwd(q[:, t:t + 1], kc, vc, lens, k[:, t:t + 1], v[:, t:t + 1],
                                            causal=causal, window=window, scale=0.6)
        lens += 1
        # A single new query attends as the last row of the full sequence only
        # when the mask has no look-ahead: its "future" keys are not cached yet.
        if causal or window[1] == 0:
            assert _close(o[:, 0], o_full[:, t]) and _close(lse[:, :, 0], lse_full[:, :, t])
    assert np.array_equal(kc[:, :n], k) and np.array_equal(vc[:, :n], v)
    assert np.isnan(kc[:, n:]).all()


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (True, (3, -1)), (True, (0, 0))])
def test_chunked_prefill_equals_full_attention(causal, window):
    rng = np.random.default_rng(2)
    n, hq, hkv, d, cap = 11, 2, 1, 4, 16
    q, k, v = _rand((1, n, hq, d), rng), _rand((1, n, hkv, d), rng), _rand((1, n, hkv, d), rng)
    o_full, lse_full = oracle.attention_fwd(q, k, v, causal=causal, window=window)
    kc = np.zeros((1, cap, hkv, d))
    vc = np.zeros((1, cap, hkv, d))
    t = 0
    for c in (4, 1, 3, 3):
        o, lse, kc, vc = oracle.kvcache_fwd(q[:, t:t + c], kc, vc, np.array([t]), k[:, t:t + c], v[:, t:t + c],
                                            causal=causal, window=window)
        assert _close(o, o_full[:, t:t + c]) and _close(lse, lse_full[:, :, t:t + c])
        t += c
    assert t == n


CASES = [
    # (B, Nq, Hq, Hkv, d, cap, lens, append)
    (2, 1, 4, 2, 3, 7, [3, 0], True),
    (2, 3, 2, 1, 4, 6, [2, 5], True),        # second entry overflows the capacity
    (3, 2, 2, 2, 2, 5, [5, 7, -2], True),    # full cache, length past capacity, negative length
    (2, 2, 4, 1, 3, 6, [4, 1], False),       # no append: attend to the valid prefix only
    (1, 4, 2, 2, 3, 8, [0], False),          # empty cache: nothing to see
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("causal,window", MASKS)
def test_matches_brute_force(case, causal, window):
    nb, nq, hq, hkv, d, cap, lens, append = case
    rng = np.random.default_rng(hash((str(case), causal, window)) % (2**32))
    q = _rand((nb, nq, hq, d), rng)
    kc, vc = _rand((nb, cap, hkv, d), rng), _rand((nb, cap, hkv, d), rng)
    kn, vn = (_rand((nb, nq, hkv, d), rng), _rand((nb, nq, hkv, d), rng)) if append else (None, None)
    o, lse, _, _ = oracle.kvcache_fwd(q, kc, vc, lens, kn, vn, causal=causal, window=window, scale=0.9)
    o_bf, lse_bf = brute_decode(q, kc, vc, lens, kn, vn, causal, window, 0.9)
    assert _close(o, o_bf) and _close(lse, lse_bf)


def test_rows_past_the_valid_length_are_never_read():
    rng = np.random.default_rng(3)
    q = _rand((2, 2, 2, 4), rng)
    kc, vc = _rand((2, 10, 1, 4), rng), _rand((2, 10, 1, 4), rng)
    kn, vn = _rand((2, 2, 1, 4), rng), _rand((2, 2, 1, 4), rng)
    lens = np.array([3, 6])
    o, lse, kc1, vc1 = oracle.kvcache_fwd(q, kc, vc, lens, kn, vn, causal=True)
    kc_nan, vc_nan = kc.copy(), vc.copy()
    for b, n in enumerate(lens):
        kc_nan[b, n:] = np.nan
        vc_nan[b, n:] = np.nan
    o2, lse2, kc2, vc2 = oracle.kvcache_fwd(q, kc_nan, vc_nan, lens, kn, vn, causal=True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # The append wrote rows n, n+1 of each entry and nothing else.
    for b, n in enumerate(lens):
        assert np.array_equal(kc1[b, n:n + 2], kn[b]) and np.array_equal(vc1[b, n:n + 2], vn[b])
        assert np.array_equal(kc1[b, :n], kc[b, :n]) and np.array_equal(kc1[b, n + 2:], kc[b, n + 2:])
        assert np.isnan(kc2[b, n + 2:]).all()


def test_batch_entries_are_independent():
    rng = np.random.default_rng(4)
    q = _rand((3, 2, 4, 3), rng)
    kc, vc = _rand((3, 9, 2, 3), rng), _rand((3, 9, 2, 3), rng)
    kn, vn = _rand((3, 2, 2, 3), rng), _rand((3, 2, 2, 3), rng)
    lens = np.array([0, 4, 8])
    o, lse, kc1, _ = oracle.kvcache_fwd(q, kc, vc, lens, kn, vn, causal=True, window=(3, -1))
    for b in range(3):
        ob, lb, kb, _ = oracle.kvcache_fwd(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], lens[b:b + 1], kn[b:b + 1],
                                           vn[b:b + 1], causal=True, window=(3, -1))
        assert np.array_equal(ob[0], o[b]) and np.array_equal(lb[0], lse[b]) and np.array_equal(kb[0], kc1[b])


def test_single_query_against_the_cache_is_a_weighted_mean():
    # Nq = 1, no mask: o = sum_j w_j v_j with w = softmax(scale q.k_j) over the
    # valid rows; with all keys equal the weights are uniform.
    rng = np.random.default_rng(5)
    kc = np.broadcast_to(_rand((1, 1, 1, 4), rng), (1, 6, 1, 4)).copy()
    vc = _rand((1, 6, 1, 4), rng)
    q = _rand((1, 1, 3, 4), rng)
    o, lse, _, _ = oracle.kvcache_fwd(q, kc, vc, [5], scale=0.5)
    for h in range(3):
        assert np.allclose(o[0, 0, h], vc[0, :5, 0].mean(axis=0), rtol=1e-13, atol=1e-13)
        assert math.isclose(lse[0, h, 0], 0.5 * float(q[0, 0, h] @ kc[0, 0, 0]) + math.log(5), rel_tol=1e-13)


# --------------------------------------------------------------------------
# Planted mistakes.
# --------------------------------------------------------------------------
MUTATIONS = [
    ("append one row late", "kc[b, length:length + n_in] = ", "kc[b, length + 1:length + 1 + n_in] = "),
    ("new rows not counted", "lk = length + n_in", "lk = length"),
    ("capacity ignored", "n_in = max(0, min(nq, cap - length))", "n_in = nq"),
    ("whole cache attended", "kc[b:b + 1, :lk], vc[b:b + 1, :lk]", "kc[b:b + 1], vc[b:b + 1]"),
    ("negative length not clamped", "length = int(min(max(lens[b], 0), cap))", "length = int(min(lens[b], cap))"),
    ("values from the key cache", "vc[b, length:length + n_in] = np.asarray(v_new)",
     "vc[b, length:length + n_in] = np.asarray(k_new)"),
]


def _mutant(old, new):
    src = inspect.getsource(KV)
    assert src.count(old) == 1, old
    src = src.replace(old, new).replace("from .attention import attention_fwd", "")
    mod = types.ModuleType("kv_mutant")
    mod.__dict__["attention_fwd"] = oracle.attention_fwd
    exec(compile(src, "kv_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(m):
    for case in CASES:
        nb, nq, hq, hkv, d, cap, lens, append = case
        rng = np.random.default_rng(77)
        q = _rand((nb, nq, hq, d), rng)
        kc, vc = _rand((nb, cap, hkv, d), rng), _rand((nb, cap, hkv, d), rng)
        kn, vn = (_rand((nb, nq, hkv, d), rng), _rand((nb, nq, hkv, d), rng)) if append else (None, None)
        for causal, window in MASKS[:3]:
            o, lse, _, _ = m.kvcache_fwd(q, kc, vc, lens, kn, vn, causal=causal, window=window, scale=0.9)
            o_bf, lse_bf = brute_decode(q, kc, vc, lens, kn, vn, causal, window, 0.9)
            if not (_close(o, o_bf) and _close(lse, lse_bf)):
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


# --------------------------------------------------------------------------
# Paged caches.
# --------------------------------------------------------------------------
def _pages_of(kc, ps):
    """Contiguous (B, cap, H, d) cache -> pages (B * cap / ps, ps, H, d), identity table."""
    nb, cap = kc.shape[:2]
    pages = kc.reshape(nb * (cap // ps), ps, *kc.shape[2:])
    return pages, np.arange(nb * (cap // ps)).reshape(nb, cap // ps)


def test_paged_with_identity_table_equals_contiguous():
    rng = np.random.default_rng(21)
    q = _rand((2, 3, 4, 3), rng)
    kc, vc = _rand((2, 8, 2, 3), rng), _rand((2, 8, 2, 3), rng)
    kn, vn = _rand((2, 3, 2, 3), rng), _rand((2, 3, 2, 3), rng)
    lens = np.array([2, 6])
    o, lse, kc1, vc1 = oracle.kvcache_fwd(q, kc, vc, lens, kn, vn, causal=True)
    kp, bt = _pages_of(kc, 4)
    vp, _ = _pages_of(vc, 4)
    o2, lse2, kp1, vp1 = oracle.kvcache_fwd_paged(q, kp, vp, lens, bt, kn, vn, causal=True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    assert np.array_equal(kp1.reshape(kc1.shape), kc1) and np.array_equal(vp1.reshape(vc1.shape), vc1)


def test_paged_table_order_and_append_placement():
    # Scattering the pages through a permuted table changes nothing but where
    # the rows live; the appended rows land in the pages the table names and
    # no other page changes.
    rng = np.random.default_rng(22)
    nb, per, ps, h, d = 3, 3, 4, 1, 2
    q = _rand((nb, 2, 2, d), rng)
    kc, vc = _rand((nb, per * ps, h, d), rng), _rand((nb, per * ps, h, d), rng)
    kn, vn = _rand((nb, 2, h, d), rng), _rand((nb, 2, h, d), rng)
    lens = np.array([3, 7, 10])
    o, lse, kc1, _ = oracle.kvcache_fwd(q, kc, vc, lens, kn, vn, causal=True, window=(2, -1))
    perm = rng.permutation(nb * per + 2)          # two spare pages
    bt = perm[:nb * per].reshape(nb, per)
    kp = _rand((nb * per + 2, ps, h, d), rng)
    vp = _rand((nb * per + 2, ps, h, d), rng)
    for b in range(nb):
        for p in range(per):
            kp[bt[b, p]] = kc[b, p * ps:(p + 1) * ps]
            vp[bt[b, p]] = vc[b, p * ps:(p + 1) * ps]
    o2, lse2, kp1, _ = oracle.kvcache_fwd_paged(q, kp, vp, lens, bt, kn, vn, causal=True, window=(2, -1))
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    for b in range(nb):
        for r in range(lens[b], lens[b] + 2):
            assert np.array_equal(kp1[bt[b, r // ps], r % ps], kn[b, r - lens[b]])
    spare = perm[nb * per:]
    assert np.array_equal(kp1[spare], kp[spare])
    changed = {(int(bt[b, r // ps])) for b in range(nb) for r in range(lens[b], lens[b] + 2)}
    for pg in set(range(nb * per)) - changed:
        assert np.array_equal(kp1[pg], kp[pg])
