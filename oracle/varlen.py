"""Attention over packed variable-length batches, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke check
and the CPU-baseline leg of the benchmark may call this module.

[P4] "FlashAttention 实战指南", section "上手 FlashAttention 的三步走": when the
sequences of a batch have different lengths, the varlen interfaces take them
packed instead of padded.  Reading (listed in the design doc): sequence b is rows
cu_q[b] .. cu_q[b+1]-1 of the packed q (total_q, Hq, d) and rows
cu_k[b] .. cu_k[b+1]-1 of the packed k, v (total_k, Hkv, d); each sequence is
attended on its own, exactly as one batch entry of :func:`attention_fwd` with its
own lengths (so masks align its last query with its own last key).  The
log-sum-exp is returned as (Hq, total_q).  Rows outside every sequence are
left at zero.

Each function is a loop over the sequences calling the fixed-length oracle on
that sequence's rows; nothing else.
"""

import numpy as np

from .attention import _as_f64, attention_bwd, attention_fwd


def _ranges(cu_q, cu_k, total_q, total_k):
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    if cu_q.ndim != 1 or cu_q.shape != cu_k.shape or cu_q.size < 1:
        raise ValueError("cu_seqlens_q / cu_seqlens_k must be 1-D with batch + 1 entries each")
    if cu_q[0] != 0 or cu_k[0] != 0 or np.any(np.diff(cu_q) < 0) or np.any(np.diff(cu_k) < 0):
        raise ValueError("offsets must start at 0 and be nondecreasing")
    if cu_q[-1] > total_q or cu_k[-1] > total_k:
        raise ValueError("offsets exceed the packed tensors")
    return [(int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])) for b in range(cu_q.size - 1)]


def _seq_slopes(alibi_slopes, b):
    if alibi_slopes is None:
        return None
    a = np.asarray(alibi_slopes, dtype=np.float64)
    return a if a.ndim == 1 else a[b]


def attention_fwd_varlen(q, k, v, cu_q, cu_k, causal=False, window=(-1, -1), scale=None, alibi_slopes=None,
                         softcap=0.0):
    """Returns (o (total_q, Hq, d), lse (Hq, total_q)) in float64.  alibi_slopes is
    (Hq,) or (batch, Hq), indexed by sequence."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    total_q, hq, d = q.shape
    o = np.zeros(q.shape)
    lse = np.zeros((hq, total_q))
    for b, (q0, q1, k0, k1) in enumerate(_ranges(cu_q, cu_k, total_q, k.shape[0])):
        ob, lb = attention_fwd(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], causal=causal, window=window,
                               scale=scale, alibi_slopes=_seq_slopes(alibi_slopes, b), softcap=softcap)
        o[q0:q1] = ob[0]
        lse[:, q0:q1] = lb[0]
    return o, lse


def attention_bwd_varlen(do, q, k, v, cu_q, cu_k, causal=False, window=(-1, -1), scale=None, alibi_slopes=None,
                         softcap=0.0):
    """Gradients (dq, dk, dv) of L = sum(O * dO) for every sequence, packed."""
    do, q, k, v = _as_f64(do), _as_f64(q), _as_f64(k), _as_f64(v)
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b, (q0, q1, k0, k1) in enumerate(_ranges(cu_q, cu_k, q.shape[0], k.shape[0])):
        g = attention_bwd(do[None, q0:q1], q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], causal=causal,
                          window=window, scale=scale, alibi_slopes=_seq_slopes(alibi_slopes, b), softcap=softcap)
        dq[q0:q1], dk[k0:k1], dv[k0:k1] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv


ALL_FUNCTIONS = (attention_fwd_varlen, attention_bwd_varlen)
