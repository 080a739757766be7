"""Seeded random configurations against the float64 oracle, through the C ABI.

Each case draws the dtype, head size, batch, query and key lengths (Nq and Nk
independent), the GQA ratio, the mask mode (none, causal, a window of random
extent on either side, causal plus a left window), an explicit scale and the
score modifiers (ALiBi slopes per head or per batch entry, softcap) from its
own seed, then checks the forward (O, LSE) and the backward (dQ, dK, dV) with
the tolerances of the structured sweeps.  It complements those sweeps with
combinations none of them lists.
"""

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import exact_tiled_attention_07_amd as fa  # noqa: E402
import oracle  # noqa: E402
from exact_tiled_attention_07_amd.workloads import random_qkv  # noqa: E402
from gpu_util import TOL, assert_close, f64  # noqa: E402

N_CASES = 40


def _draw(i):
    rng = np.random.default_rng(7000 + i)
    dtype = str(rng.choice(["fp16", "bf16", "fp32"]))
    if dtype == "fp32":
        d = int(rng.choice([4, 12, 32, 64, 100, 128]))
    else:
        d = int(rng.choice([8, 24, 64, 64, 96, 128, 128]))
    b = int(rng.integers(1, 4))
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    nq = int(rng.integers(1, 300))
    nk = int(rng.integers(1, 300))
    mode = int(rng.integers(0, 4))
    kw = {}
    if mode == 1:
        kw["causal"] = True
    elif mode == 2:
        kw["window_size"] = (int(rng.integers(-1, 80)), int(rng.integers(-1, 80)))
    elif mode == 3:
        kw["causal"] = True
        kw["window_size"] = (int(rng.integers(0, 80)), -1)
    if rng.random() < 0.3:
        kw["scale"] = float(rng.uniform(0.02, 0.3))
    slopes = None
    if rng.random() < 0.25:
        base = np.array([2.0 ** (-8.0 * (h + 1) / hq) for h in range(hq)])
        slopes = (np.stack([base * (1.0 + 0.5 * rng.random()) for _ in range(b)]) if rng.random() < 0.5
                  else base).astype(np.float32)
    softcap = float(rng.uniform(0.5, 4.0)) if rng.random() < 0.25 else 0.0
    return dtype, d, b, hq, hkv, nq, nk, kw, slopes, softcap


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    dtype, d, b, hq, hkv, nq, nk, kw, slopes, softcap = _draw(i)
    print(f"case {i}: {dtype} d={d} B={b} Hq={hq} Hkv={hkv} Nq={nq} Nk={nk} {kw} "
          f"alibi={'none' if slopes is None else slopes.shape} softcap={softcap}", flush=True)
    sys.stdout.flush()
    q, _, _, do = random_qkv((b, nq, hq, d), (b, nq, hkv, d), dtype, seed=7100 + i)
    _, k, v, _ = random_qkv((b, nk, hq, d), (b, nk, hkv, d), dtype, seed=7200 + i)
    sl_d = torch.from_numpy(slopes).cuda() if slopes is not None else None
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, alibi_slopes=sl_d, softcap=softcap, **kw)
    dq, dk, dv = fa.bwd(dod, qd, kd, vd, o, lse, alibi_slopes=sl_d, softcap=softcap, **kw)
    torch.cuda.synchronize()
    okw = dict(causal=kw.get("causal", False), window=tuple(kw.get("window_size", (-1, -1))), scale=kw.get("scale"),
               alibi_slopes=None if slopes is None else slopes.astype(np.float64), softcap=softcap)
    o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), **okw)
    g_ref = oracle.attention_bwd(f64(do), f64(q), f64(k), f64(v), **okw)
    tol = TOL[q.dtype]
    assert_close(o, o_ref, tol, "O")
    assert_close(lse, lse_ref, tol, "LSE")
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        assert_close(got, ref, 2 * tol, name)


def _mask(rng):
    mode = int(rng.integers(0, 3))
    if mode == 1:
        return {"causal": True}
    if mode == 2:
        return {"window_size": (int(rng.integers(-1, 60)), int(rng.integers(-1, 60)))}
    return {}


def _okw(kw, slopes, softcap):
    return dict(causal=kw.get("causal", False), window=tuple(kw.get("window_size", (-1, -1))), scale=kw.get("scale"),
                alibi_slopes=None if slopes is None else slopes.astype(np.float64), softcap=softcap)


@pytest.mark.parametrize("i", range(12))
def test_random_packed_batch(i):
    # Packed batches: random sequence counts and lengths (empty sequences included).
    rng = np.random.default_rng(7300 + i)
    dtype = str(rng.choice(["fp16", "bf16"]))
    d = int(rng.choice([64, 128, 40]))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 4]))
    nseq = int(rng.integers(1, 6))
    lq = [int(x) for x in rng.integers(0, 200, nseq)]
    lk = [int(x) for x in rng.integers(0, 200, nseq)]
    kw = _mask(rng)
    softcap = float(rng.uniform(1.0, 3.0)) if rng.random() < 0.3 else 0.0
    print(f"packed case {i}: {dtype} d={d} Hq={hq} Hkv={hkv} lq={lq} lk={lk} {kw} softcap={softcap}", flush=True)
    dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]
    g = torch.Generator("cpu").manual_seed(7400 + i)
    tq, tk = sum(lq), sum(lk)
    q = torch.randn((tq, hq, d), generator=g).to(dt)
    k = torch.randn((tk, hkv, d), generator=g).to(dt)
    v = torch.randn((tk, hkv, d), generator=g).to(dt)
    do = torch.randn((tq, hq, d), generator=g).to(dt)
    cu_q = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(lk)), dtype=torch.int32)
    qd, kd, vd, dod, cq, ck = (t.cuda() for t in (q, k, v, do, cu_q, cu_k))
    mq, mk = max(lq), max(lk)
    o, lse = fa.fwd_varlen(qd, kd, vd, cq, ck, mq, mk, softcap=softcap, **kw)
    dq, dk, dv = fa.bwd_varlen(dod, qd, kd, vd, o, lse, cq, ck, mq, mk, softcap=softcap, **kw)
    torch.cuda.synchronize()
    okw = _okw(kw, None, softcap)
    o_ref, lse_ref = oracle.attention_fwd_varlen(f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(), **okw)
    g_ref = oracle.attention_bwd_varlen(f64(do), f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(), **okw)
    tol = TOL[dt]
    assert_close(o, o_ref, tol, "O")
    assert_close(lse, lse_ref, tol, "LSE")
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        assert_close(got, ref, 2 * tol, name)


@pytest.mark.parametrize("i", range(12))
def test_random_kvcache(i):
    # Decode / chunked prefill against a ragged cache: random lengths, new-token
    # counts, split counts, masks and modifiers; contiguous and through pages.
    rng = np.random.default_rng(7500 + i)
    dtype = str(rng.choice(["fp16", "bf16"]))
    d = int(rng.choice([64, 128, 96]))
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 8]))
    b = int(rng.integers(1, 4))
    nq = int(rng.choice([1, 1, 2, 5, 17]))
    cap = 64 * int(rng.integers(2, 12))
    lens = [int(x) for x in rng.integers(0, cap - nq + 1, b)]
    kw = {"causal": True} if rng.random() < 0.6 else _mask(rng)
    splits = int(rng.choice([0, 0, 1, 3, 7]))
    softcap = float(rng.uniform(1.0, 3.0)) if rng.random() < 0.3 else 0.0
    print(f"kvcache case {i}: {dtype} d={d} B={b} Hq={hq} Hkv={hkv} Nq={nq} cap={cap} lens={lens} {kw} "
          f"splits={splits} softcap={softcap}", flush=True)
    dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]
    g = torch.Generator("cpu").manual_seed(7600 + i)
    q = torch.randn((b, nq, hq, d), generator=g).to(dt)
    kc = torch.randn((b, cap, hkv, d), generator=g).to(dt)
    vc = torch.randn((b, cap, hkv, d), generator=g).to(dt)
    kn = torch.randn((b, nq, hkv, d), generator=g).to(dt)
    vn = torch.randn((b, nq, hkv, d), generator=g).to(dt)
    lensd = torch.tensor(lens, dtype=torch.int32, device="cuda")
    kcd, vcd = kc.cuda(), vc.cuda()
    o, lse = fa.fwd_kvcache(q.cuda(), kcd, vcd, lensd, kn.cuda(), vn.cuda(), num_splits=splits, softcap=softcap, **kw)
    torch.cuda.synchronize()
    okw = _okw(kw, None, softcap)
    o_ref, lse_ref, kc_ref, vc_ref = oracle.kvcache_fwd(f64(q), f64(kc), f64(vc), np.array(lens), f64(kn), f64(vn),
                                                        **okw)
    assert_close(o, o_ref, TOL[dt], "O")
    assert_close(lse, lse_ref, TOL[dt], "LSE")
    assert np.array_equal(f64(kcd), kc_ref) and np.array_equal(f64(vcd), vc_ref)
    # The same through 64-row pages in a shuffled pool.
    npg = b * cap // 64
    perm = torch.from_numpy(rng.permutation(npg).astype(np.int64))
    kp = torch.empty((npg, 64, hkv, d), dtype=dt)
    vp = torch.empty((npg, 64, hkv, d), dtype=dt)
    kp[perm] = kc.reshape(npg, 64, hkv, d)
    vp[perm] = vc.reshape(npg, 64, hkv, d)
    table = perm.to(torch.int32).reshape(b, cap // 64).cuda()
    kpd, vpd = kp.cuda(), vp.cuda()
    o2, lse2 = fa.fwd_kvcache_paged(q.cuda(), kpd, vpd, lensd, table, kn.cuda(), vn.cuda(), num_splits=splits,
                                    softcap=softcap, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
