"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, run the float64 oracle on the same CPU inputs, and compare."""

import json
import os

import numpy as np
import torch

import exact_tiled_attention_07_amd as fa
import oracle
from compare import describe, within

# Max-abs tolerances of the HIP path against the float64 oracle: O and LSE
# use the first, dQ/dK/dV twice it.
TOL = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 1.6e-2}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def max_err(got, ref):
    """Max |got - ref| over finite reference entries; -inf entries must match exactly."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), "-inf pattern differs"
    fin = ~inf_ref
    assert np.all(np.isfinite(got[fin])), "non-finite values in the GPU result"
    return float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0


DTYPE_NAME = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}


def record_errors(case, errors):
    """Appends {case, output: statistics} as one JSON line to the file named by
    FA_PARITY_LOG, if set (the literal max-abs errors of the full-size runs)."""
    path = os.environ.get("FA_PARITY_LOG")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps({"case": case, **{k: {kk: (None if vv == float("inf") else vv) for kk, vv in v.items()}
                                             for k, v in errors.items()}}) + "\n")


def assert_close(got, ref, tol, what):
    """Oracle comparison rule of compare.py for a GPU tensor against a float64 array."""
    ok, info = within(f64(got), ref, DTYPE_NAME[got.dtype], tol)
    info = dict(info, tol=tol)
    assert ok, f"{what}: {describe(info, tol)}"
    return info


def gpu_fwd(q, k, v, **kw):
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), **kw)
    torch.cuda.synchronize()
    return o, lse


def gpu_bwd(do, q, k, v, o, lse, **kw):
    dq, dk, dv = fa.bwd(do.cuda(), q.cuda(), k.cuda(), v.cuda(), o, lse, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


def oracle_kw(kw):
    return dict(causal=kw.get("causal", False), window=tuple(kw.get("window_size", (-1, -1))),
                scale=kw.get("scale"))


def check_fwd(q, k, v, tol_mult=1.0, **kw):
    o, lse = gpu_fwd(q, k, v, **kw)
    o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), **oracle_kw(kw))
    tol = TOL[q.dtype] * tol_mult
    eo = assert_close(o, o_ref, tol, "O")
    el = assert_close(lse, lse_ref, tol, "LSE")
    return o, lse, eo, el


def check_bwd(q, k, v, do, **kw):
    o, lse = gpu_fwd(q, k, v, **kw)
    dq, dk, dv = gpu_bwd(do, q, k, v, o, lse, **kw)
    ref = oracle.attention_bwd(f64(do), f64(q), f64(k), f64(v), **oracle_kw(kw))
    tol = 2 * TOL[q.dtype]
    errs = {}
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        errs[name] = assert_close(got, r, tol, name)
    return errs
