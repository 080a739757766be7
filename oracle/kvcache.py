"""Attention against a KV cache (incremental decoding), in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke check
and the CPU-baseline leg of the benchmark may call this module.

[P4] "FlashAttention 实战指南", section "增量解码场景flash_attn_with_kvcache": for
decoding a few tokens per step, the new keys and values are appended to an
existing cache and attention is computed in place; cache_seqlens marks each batch
entry's valid cache length; num_splits divides the key range (a scheduling
choice that does not change the result, so it has no counterpart here).
[P5] "AI模型推理优化Flash Attention原理", section "实际怎么用": its KV-cache class
writes the new rows at the current position, advances the position by their
count and hands back the cache prefix up to it -- the append step below.

Readings taken where the section leaves a step open (each is listed in the design doc):

* the new rows of batch entry b land at cache rows L_b .. L_b + Nq - 1, where
  L_b = cache_seqlens[b] is the length before the append; rows that would fall
  past the cache capacity are dropped, and lengths outside [0, capacity] are
  clamped to it;
* the queries then see the first Lk_b = min(L_b + Nq, capacity) cache rows (L_b
  when nothing is appended), with the same causal / window rule as the main
  path and the last query aligned to the last key, exactly as
  :func:`oracle.attention.attention_fwd` does for seqlen_k = Lk_b.

Step order: the append, then :func:`attention_fwd` on each batch entry's valid
prefix.  Nothing is tiled, split or merged.
"""

import numpy as np

from .attention import attention_fwd


def _entry_slopes(alibi_slopes, b):
    """Slopes of batch entry b as a (nheads_q,) array (None stays None)."""
    if alibi_slopes is None:
        return None
    a = np.asarray(alibi_slopes, dtype=np.float64)
    return a if a.ndim == 1 else a[b]


def kvcache_fwd(q, k_cache, v_cache, cache_seqlens, k_new=None, v_new=None, causal=False, window=(-1, -1),
                scale=None, alibi_slopes=None, softcap=0.0):
    """Append, then attend.

    q (B, Nq, Hq, d); k_cache, v_cache (B, capacity, Hkv, d); cache_seqlens (B,)
    integers; k_new, v_new (B, Nq, Hkv, d) or both None; alibi_slopes and softcap
    as in :func:`oracle.attention.attention_fwd`.
    Returns (o (B, Nq, Hq, d), lse (B, Hq, Nq), k_cache_after, v_cache_after):
    o and lse in float64, the caches as copies in their input dtype.
    """
    q = np.asarray(q)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    b_, nq, hq, d = q.shape
    cap = kc.shape[1]
    if kc.shape != vc.shape or kc.shape[0] != b_ or kc.shape[3] != d:
        raise ValueError("caches must be (batch, capacity, nheads_kv, headdim)")
    lens = np.asarray(cache_seqlens, dtype=np.int64)
    if lens.shape != (b_,):
        raise ValueError("cache_seqlens must have one entry per batch entry")
    o = np.zeros((b_, nq, hq, d))
    lse = np.zeros((b_, hq, nq))
    for b in range(b_):
        length = int(min(max(lens[b], 0), cap))
        if k_new is not None:
            n_in = max(0, min(nq, cap - length))
            kc[b, length:length + n_in] = np.asarray(k_new)[b, :n_in]
            vc[b, length:length + n_in] = np.asarray(v_new)[b, :n_in]
            lk = length + n_in
        else:
            lk = length
        ob, lb = attention_fwd(q[b:b + 1], kc[b:b + 1, :lk], vc[b:b + 1, :lk], causal=causal, window=window,
                               scale=scale, alibi_slopes=_entry_slopes(alibi_slopes, b), softcap=softcap)
        o[b] = ob[0]
        lse[b] = lb[0]
    return o, lse, kc, vc


def kvcache_fwd_paged(q, k_pages, v_pages, cache_seqlens, block_table, k_new=None, v_new=None, causal=False,
                      window=(-1, -1), scale=None, alibi_slopes=None, softcap=0.0):
    """The same computation over a paged cache ([P4] section "增量解码场景
    flash_attn_with_kvcache": block_table turns on a cache stored in blocks).

    k_pages, v_pages (num_pages, page_size, Hkv, d); block_table (B, pages per
    entry) integers, clamped to [0, num_pages).  Reading: row j of entry b is
    row j % page_size of page block_table[b, j // page_size]; the capacity of
    an entry is its pages times page_size.  Steps: gather each entry's pages
    into a contiguous cache, run :func:`kvcache_fwd`, write the pages back.
    Returns (o, lse, k_pages_after, v_pages_after).
    """
    kp = np.array(k_pages, copy=True)
    vp = np.array(v_pages, copy=True)
    bt = np.clip(np.asarray(block_table, dtype=np.int64), 0, kp.shape[0] - 1)
    nb, per = bt.shape
    ps = kp.shape[1]
    kc = np.stack([np.concatenate([kp[bt[b, p]] for p in range(per)]) for b in range(nb)])
    vc = np.stack([np.concatenate([vp[bt[b, p]] for p in range(per)]) for b in range(nb)])
    o, lse, kc, vc = kvcache_fwd(q, kc, vc, cache_seqlens, k_new, v_new, causal=causal, window=window, scale=scale,
                                 alibi_slopes=alibi_slopes, softcap=softcap)
    for b in range(nb):
        for p in range(per):
            kp[bt[b, p]] = kc[b, p * ps:(p + 1) * ps]
            vp[bt[b, p]] = vc[b, p * ps:(p + 1) * ps]
    return o, lse, kp, vp


ALL_FUNCTIONS = (kvcache_fwd, kvcache_fwd_paged)
