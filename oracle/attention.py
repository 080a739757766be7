"""Plain float64 attention: forward (O and per-row logsumexp) and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke check
and the CPU-baseline leg of the benchmark may call this module.

Tensor layout follows [P4] "FlashAttention 实战指南", section "上手 FlashAttention 的
三步走": q is (batch, seqlen_q, nheads_q, headdim); k and v are
(batch, seqlen_k, nheads_kv, headdim).  The log-sum-exp output is
(batch, nheads_q, seqlen_q).

Readings taken where the pages leave a step open (each is listed in the design doc):

* scale multiplies Q K^T before the mask and the softmax; the default is
  1/sqrt(headdim) ([P5] section "先搞清楚原理");
* window_size (left, right) is inclusive: key j is visible from query i iff
  i' - left <= j <= i' + right, where a negative bound is unbounded ([P4] section
  "进阶参数如何配置causal、window_size 与 MQA/GQA") and i' = i + (seqlen_k - seqlen_q)
  aligns the last query with the last key (bottom-right alignment);
* causal is an additional "j <= i'" condition, combined with the window by AND;
* MQA/GQA: query head h reads K/V head floor(h / G), G = nheads_q / nheads_kv
  (contiguous groups) ([P4] same section);
* a query row that sees no key gets O = 0, LSE = -inf and zero gradients;
* the backward is the exact derivative of the forward (the pages only say that
  the backward recomputes the attention matrix, [P4] section
  "长序列注意力为什么会爆内存").
"""

import math

import numpy as np

# Per-array memory budget for one row block of the score matrix (bytes).
_ROW_BLOCK_BYTES = 128 << 20


def _as_f64(x):
    """Upcast to float64 (exact for fp32, fp16 and bf16 values)."""
    return np.asarray(x, dtype=np.float64)


def head_of(h, nheads_q, nheads_kv):
    """K/V head read by query head ``h``.

    [P4] section "进阶参数如何配置causal、window_size 与 MQA/GQA": K and V may have
    fewer heads than Q, as long as the Q head count is an integer multiple of the
    K/V head count.  Reading: consecutive query heads share one K/V head.
    """
    if nheads_q % nheads_kv != 0:
        raise ValueError("nheads_q must be a multiple of nheads_kv")
    return h // (nheads_q // nheads_kv)


def visible(seqlen_q, seqlen_k, causal=False, window=(-1, -1), rows=None):
    """Boolean (len(rows), seqlen_k) visibility of key j from query i.

    [P4] section "上手 FlashAttention 的三步走" (causal for autoregressive use) and
    section "进阶参数如何配置causal、window_size 与 MQA/GQA" (window (left, right),
    -1 unbounded).  Queries are aligned to the end of the keys.
    """
    wl, wr = window
    if wl < -1 or wr < -1:
        raise ValueError("window bounds must be >= -1")
    if rows is None:
        rows = np.arange(seqlen_q)
    i = np.asarray(rows, dtype=np.int64)[:, None] + (seqlen_k - seqlen_q)
    j = np.arange(seqlen_k, dtype=np.int64)[None, :]
    vis = np.ones((i.shape[0], seqlen_k), dtype=bool)
    if causal:
        vis &= j <= i
    if wl >= 0:
        vis &= j >= i - wl
    if wr >= 0:
        vis &= j <= i + wr
    return vis


def scores(q_rows, k_head, scale):
    """S = scale * Q K^T for one head: (R, d) x (Nk, d) -> (R, Nk).

    [P5] section "先搞清楚原理" (scores are Q times K transposed, divided by
    sqrt(d)); [P4] section "长序列注意力为什么会爆内存" (first of the three steps).
    """
    return scale * (_as_f64(q_rows) @ _as_f64(k_head).T)


def masked_softmax(s, vis):
    """Row softmax over visible keys: returns (P, lse).

    [P4] section "长序列注意力为什么会爆内存" (second step: softmax of each score
    row).  Hidden entries are -inf; the row maximum is subtracted before exp (a
    no-op in exact arithmetic that keeps exp from overflowing).  lse is the
    natural-log log-sum-exp of the visible scores; an empty row gives P = 0,
    lse = -inf.
    """
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    total = e.sum(axis=1)
    denom = np.where(empty, 1.0, total)
    p = e / denom[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    return p, lse


def slope_of(alibi_slopes, b, h):
    """ALiBi slope of (batch b, query head h): alibi_slopes is None, (nheads_q,)
    (the same for every batch entry) or (batch, nheads_q)."""
    if alibi_slopes is None:
        return None
    a = np.asarray(alibi_slopes, dtype=np.float64)
    return float(a[h] if a.ndim == 1 else a[b, h])


def modified_logits(x, rows, seqlen_q, seqlen_k, slope=None, softcap=0.0):
    """Score modifiers of [P4] section "进阶参数如何配置causal、window_size 与 MQA/GQA":
    softcap truncates the logits to [-softcap, softcap]; alibi_slopes is a
    positional bias that decays a score with the distance between query and key.

    Readings (listed in the design doc): the logits are the scaled scores x = scale * q.k;
    the truncation is a clamp, applied first; the ALiBi bias is
    -slope * |i' - j| with i' = i + seqlen_k - seqlen_q (the same alignment as
    the mask), added after the clamp and before the mask.
    Returns (logits, gate): gate is the derivative of the clamp, 1 where
    |x| < softcap and 0 elsewhere (all ones without softcap).
    """
    out = x
    gate = np.ones_like(x)
    if softcap > 0:
        out = np.clip(x, -softcap, softcap)
        gate = (np.abs(x) < softcap).astype(np.float64)
    if slope is not None:
        aligned = np.asarray(rows, dtype=np.int64) - seqlen_q + seqlen_k
        j = np.arange(seqlen_k, dtype=np.int64)
        out = out - slope * np.abs(aligned[:, None] - j[None, :])
    return out, gate


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be (batch, seqlen, nheads, headdim)")
    b, nq, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[3] != d:
        raise ValueError("k and v must be (batch, seqlen_k, nheads_kv, headdim)")
    if hq % k.shape[2] != 0:
        raise ValueError("nheads_q must be a multiple of nheads_kv")
    return b, nq, k.shape[1], hq, k.shape[2], d


def _row_blocks(nq, nk):
    r = max(1, _ROW_BLOCK_BYTES // max(1, 8 * nk))
    return [(i, min(nq, i + r)) for i in range(0, nq, r)]


def attention_fwd(q, k, v, causal=False, window=(-1, -1), scale=None, alibi_slopes=None, softcap=0.0):
    """O = softmax(scale Q K^T + mask) V and the per-row log-sum-exp.

    [P4] section "长序列注意力为什么会爆内存" (the three steps), [P5] section
    "先搞清楚原理" (the standard_attention definition).  The whole score row is
    materialised in float64 (row blocks only bound memory).  Optional score
    modifiers: :func:`modified_logits`.
    Returns (o, lse): o (B, Nq, Hq, d) and lse (B, Hq, Nq), both float64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b_, nq, nk, hq, hkv, d = _check(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((b_, nq, hq, d))
    lse = np.zeros((b_, hq, nq))
    for b in range(b_):
        for h in range(hq):
            g = head_of(h, hq, hkv)
            kh, vh = k[b, :, g, :], v[b, :, g, :]
            for r0, r1 in _row_blocks(nq, nk):
                rows = np.arange(r0, r1)
                s = scores(q[b, r0:r1, h, :], kh, scale)
                s, _ = modified_logits(s, rows, nq, nk, slope_of(alibi_slopes, b, h), softcap)
                p, l_ = masked_softmax(s, visible(nq, nk, causal, window, rows))
                o[b, r0:r1, h, :] = p @ vh
                lse[b, h, r0:r1] = l_
    return o, lse


def attention_fwd_rows(q, k, v, b, h, rows, causal=False, window=(-1, -1), scale=None, alibi_slopes=None,
                       softcap=0.0):
    """O and lse of selected query rows of one (batch, head): same definition as
    :func:`attention_fwd`, evaluated only where asked (for sampled checks at
    full size).  Returns (o_rows (R, d), lse_rows (R,))."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _, nq, nk, hq, hkv, d = _check(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    g = head_of(h, hq, hkv)
    s = scores(q[b, rows, h, :], k[b, :, g, :], scale)
    s, _ = modified_logits(s, rows, nq, nk, slope_of(alibi_slopes, b, h), softcap)
    p, l_ = masked_softmax(s, visible(nq, nk, causal, window, rows))
    return p @ v[b, :, g, :], l_


def attention_bwd(do, q, k, v, causal=False, window=(-1, -1), scale=None, alibi_slopes=None, softcap=0.0):
    """Gradients of L = sum(O * dO) with respect to q, k and v.

    The pages state only that the backward pass recomputes the attention matrix
    instead of storing it ([P4] section "长序列注意力为什么会爆内存"); the formulas
    are the exact derivative of :func:`attention_fwd`:

      dP = dO V^T,   D_i = sum_j P_ij dP_ij,   dS = P * (dP - D),
      dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO,

    with dK and dV summed over the query heads that share a K/V head.  With the
    score modifiers, P comes from the modified logits and dS is multiplied by
    the clamp's derivative (the ALiBi bias does not depend on q or k).
    Returns (dq, dk, dv) in float64 with the shapes of q, k, v.
    """
    do, q, k, v = _as_f64(do), _as_f64(q), _as_f64(k), _as_f64(v)
    b_, nq, nk, hq, hkv, d = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(b_):
        for h in range(hq):
            g = head_of(h, hq, hkv)
            kh, vh = k[b, :, g, :], v[b, :, g, :]
            for r0, r1 in _row_blocks(nq, nk):
                rows = np.arange(r0, r1)
                qr, dor = q[b, r0:r1, h, :], do[b, r0:r1, h, :]
                s = scores(qr, kh, scale)
                s, gate = modified_logits(s, rows, nq, nk, slope_of(alibi_slopes, b, h), softcap)
                p, _ = masked_softmax(s, visible(nq, nk, causal, window, rows))
                dp = dor @ vh.T
                dsum = np.sum(p * dp, axis=1)
                ds = p * (dp - dsum[:, None])
                ds = ds * gate
                dq[b, r0:r1, h, :] = scale * (ds @ kh)
                dk[b, :, g, :] += scale * (ds.T @ qr)
                dv[b, :, g, :] += p.T @ dor
    return dq, dk, dv


ALL_FUNCTIONS = (head_of, visible, scores, masked_softmax, slope_of, modified_logits, attention_fwd,
                 attention_fwd_rows, attention_bwd)
