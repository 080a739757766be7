"""A float64 model of the 16-bit kernels' rounding points, for stress inputs.

The fp16/bf16 kernels compute in fp32 but round three quantities to the input
type before a matrix product (the internal-precision reading: products on the
matrix cores take 16-bit operands): P before O += P V (forward) and
dV += P^T dO, and dS = P (dP - D) before dQ += dS K and dK += dS^T Q; and
D_i = sum_c dO_ic O_ic is formed from the stored (16-bit) forward output O.  This module applies exactly those
roundings to otherwise exact float64 arithmetic, so that its error against the
oracle is the error that the rounding policy alone costs.  On inputs whose
gradients are large or cancel (scores with std 4, keys that climb along the
sequence) that cost can exceed the absolute bounds; the stress tests then ask
the GPU to stay within the model's error plus a small margin, i.e. to add no
error of its own beyond the policy.

Test infrastructure: uses the oracle's mask and softmax primitives; nothing here
is imported by the library.
"""

import math

import numpy as np
import torch

import oracle

TORCH_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def round_to(x, dtype_name):
    """float64 -> the 16-bit type (round to nearest even) -> float64; None
    leaves x as it is (the model without roundings is the exact backward)."""
    if dtype_name is None:
        return np.asarray(x, dtype=np.float64)
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DT[dtype_name]).double().numpy()


def _stored_output(s, vis, vh, dtype_name):
    """The forward's output for one head: unnormalised probabilities (against
    the row maximum) rounded before the product with V, the fp32 row sum of the
    unrounded ones, the result rounded at the store."""
    m = np.max(np.where(vis, s, -np.inf), axis=1, initial=-np.inf)
    e = np.where(vis, np.exp(s - np.where(np.isfinite(m), m, 0.0)[:, None]), 0.0)
    tot = e.sum(axis=1)
    return round_to((round_to(e, dtype_name) @ vh) / np.where(tot > 0, tot, 1.0)[:, None], dtype_name)


def policy_fwd(q, k, v, dtype_name, causal=False, window=(-1, -1), scale=None):
    """O (float64, already rounded to the type) as the forward's rounding policy gives it."""
    b_, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = np.zeros_like(q)
    vis = oracle.visible(nq, nk, causal, window)
    for b in range(b_):
        for h in range(hq):
            g = oracle.head_of(h, hq, hkv)
            o[b, :, h] = _stored_output(oracle.scores(q[b, :, h], k[b, :, g], scale), vis, v[b, :, g], dtype_name)
    return o


def policy_grads(do, q, k, v, dtype_name, causal=False, window=(-1, -1), scale=None):
    """(dq, dk, dv) in float64 as the kernels' rounding policy gives them
    (before the final rounding of the outputs)."""
    b_, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    vis = oracle.visible(nq, nk, causal, window)
    for b in range(b_):
        for h in range(hq):
            g = oracle.head_of(h, hq, hkv)
            kh, vh, qh, doh = k[b, :, g], v[b, :, g], q[b, :, h], do[b, :, h]
            s = oracle.scores(qh, kh, scale)
            p, _ = oracle.masked_softmax(s, vis)
            o_stored = _stored_output(s, vis, vh, dtype_name) if dtype_name else p @ vh
            dp = doh @ vh.T
            dsum = np.sum(doh * o_stored, axis=1)
            ds = round_to(p * (dp - dsum[:, None]), dtype_name)
            dq[b, :, h] = scale * (ds @ kh)
            dk[b, :, g] += scale * (ds.T @ qh)
            dv[b, :, g] += round_to(p, dtype_name).T @ doh
    return dq, dk, dv
