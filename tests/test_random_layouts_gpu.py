"""Randomised parity over memory layouts and the 16-bit rounding bound.

It complements test_random_gpu.py (which draws the score modifiers and paged
caches): seeded draws of dtype, head dim, GQA group, lengths, mask, scale and
memory layout (contiguous, rows padded past the head dim, heads sliced out of
a wider tensor), each run through fa_fwd and fa_bwd, packed batches through
the varlen entry points, and KV-cache calls, all against the float64 oracle.

Case i draws from its own seed (10000 + i), so a failure names a case that
reruns alone (pytest -k "case_17").  Lengths stay small (at most 260) so the
oracle finishes quickly, yet cross several 32/64-row tiles with ragged tails;
head dims include ones below the kernels' 64 / 128 (zero-padded columns);
scales keep d * scale^2 within [0.25, 2].

fp32 results are held to the absolute bounds.  fp16/bf16 results are held to
the larger of the absolute bound and twice the error of the float64 model of
the kernels' rounding points (rounding_model.py): some legal shapes, e.g. many
queries against a handful of keys, sum so many rounded dS and P terms into
dK and dV that the rounding policy alone exceeds the absolute bound, and the
model then measures what that policy costs; the GPU must add nothing of its
own beyond it.  Every case records the model's error next to the GPU's.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
from compare import compare  # noqa: E402
from exact_tiled_attention_07_amd.workloads import random_qkv  # noqa: E402
from gpu_util import DTYPE_NAME, TOL, assert_close, check_bwd, check_fwd, f64, gpu_bwd, gpu_fwd  # noqa: E402
from rounding_model import policy_fwd, policy_grads, round_to  # noqa: E402

MODEL_FACTOR = 2.0


def hold(got, ref, model, dt, tol, what):
    """|got - ref| within max(tol, MODEL_FACTOR x the rounding model's error)."""
    e_gpu = compare(np.asarray(got), ref, dt, tol)
    e_model = compare(round_to(model, dt), ref, dt, tol)
    bound = max(tol, MODEL_FACTOR * e_model["raw"])
    assert e_gpu["raw"] <= bound, \
        f"{what}: max-abs {e_gpu['raw']:.3e}, rounding model {e_model['raw']:.3e} (allowed {bound:.3e})"
    return e_gpu["raw"], e_model["raw"]


def check_fwd_bwd_16(q, k, v, do, **kw):
    """Forward and backward of 16-bit inputs against the oracle, under the
    rounding-policy bound (see the module docstring)."""
    dt = DTYPE_NAME[q.dtype]
    tol = TOL[q.dtype]
    ow = dict(causal=kw.get("causal", False), window=tuple(kw.get("window_size", (-1, -1))), scale=kw.get("scale"))
    o, lse = gpu_fwd(q, k, v, **kw)
    grads = gpu_bwd(do, q, k, v, o, lse, **kw)
    qf, kf, vf, dof = f64(q), f64(k), f64(v), f64(do)
    o_ref, l_ref = oracle.attention_fwd(qf, kf, vf, **ow)
    assert_close(lse, l_ref, tol, "LSE")
    errs = {"o": hold(f64(o), o_ref, policy_fwd(qf, kf, vf, dt, **ow), dt, tol, "O")}
    ref = oracle.attention_bwd(dof, qf, kf, vf, **ow)
    model = policy_grads(dof, qf, kf, vf, dt, **ow)
    for name, got, r, m in zip(("dq", "dk", "dv"), grads, ref, model):
        errs[name] = hold(f64(got), r, m, dt, 2 * tol, name)
    print("  (gpu, model) max-abs:", {k_: (f"{a:.2e}", f"{b:.2e}") for k_, (a, b) in errs.items()}, flush=True)

CASES = 160


def draw(i):
    rng = np.random.default_rng(10_000 + i)
    dtype = str(rng.choice(["fp32", "fp16", "bf16"], p=[0.2, 0.4, 0.4]))
    if dtype == "fp32":
        d = int(rng.choice([4, 12, 20, 64, 100, 128]))
    else:
        d = int(rng.choice([8, 16, 32, 40, 64, 72, 96, 104, 128]))
    hkv = int(rng.choice([1, 2, 3]))
    g = int(rng.choice([1, 2, 4]))
    b = int(rng.integers(1, 3))
    nq, nk = int(rng.integers(1, 261)), int(rng.integers(1, 261))
    kind = str(rng.choice(["full", "causal", "window", "causal_left"]))
    mask = {}
    if kind == "causal":
        mask = dict(causal=True)
    elif kind == "window":
        mask = dict(window_size=(int(rng.integers(-1, 80)), int(rng.integers(-1, 80))))
    elif kind == "causal_left":
        mask = dict(causal=True, window_size=(int(rng.integers(0, 80)), -1))
    scale = float(np.sqrt(rng.uniform(0.25, 2.0) / d))
    layout = str(rng.choice(["contiguous", "wide_rows", "head_slice"]))
    return dict(dtype=dtype, d=d, hkv=hkv, g=g, b=b, nq=nq, nk=nk, mask=mask, scale=scale, layout=layout)


def arrange(t, layout, extra):
    """The same values on the GPU in another memory layout: rows padded past
    the head dim, or heads taken from a tensor with one more head (built on
    the device, since a copy of a strided view would come out contiguous)."""
    t = t.cuda()
    if layout == "contiguous":
        return t
    B, N, H, D = t.shape
    if layout == "wide_rows":
        w = torch.zeros(B, N, H, D + extra, dtype=t.dtype, device="cuda")
        w[..., :D] = t
        return w[..., :D]
    w = torch.zeros(B, N, H + 1, D, dtype=t.dtype, device="cuda")
    w[:, :, :H] = t
    return w[:, :, :H]


@pytest.mark.parametrize("i", range(CASES), ids=[f"case_{i}" for i in range(CASES)])
def test_random_case(i):
    c = draw(i)
    print(f"fuzz case {i}: {c}", flush=True)
    hq = c["hkv"] * c["g"]
    q, _, _, do = random_qkv((c["b"], c["nq"], hq, c["d"]), (c["b"], c["nq"], c["hkv"], c["d"]), c["dtype"], seed=i)
    _, k, v, _ = random_qkv((c["b"], c["nk"], hq, c["d"]), (c["b"], c["nk"], c["hkv"], c["d"]), c["dtype"],
                            seed=1000 + i)
    extra = 4 if c["dtype"] == "fp32" else 8  # one 16-byte chunk
    q, k, v = (arrange(t, c["layout"], extra) for t in (q, k, v))
    kw = dict(c["mask"], scale=c["scale"])
    if c["dtype"] == "fp32":
        check_fwd(q, k, v, **kw)
        check_bwd(q, k, v, do, **kw)
    else:
        check_fwd_bwd_16(q, k, v, do, **kw)


# ---------------------------------------------------------------------------
# Packed variable-length batches and KV-cache calls, drawn the same way.
# ---------------------------------------------------------------------------
VARLEN_CASES = 40
KV_CASES = 40


def draw_varlen(i):
    rng = np.random.default_rng(20_000 + i)
    dtype = str(rng.choice(["fp32", "fp16", "bf16"], p=[0.2, 0.4, 0.4]))
    d = int(rng.choice([8, 20, 64, 100]) if dtype == "fp32" else rng.choice([16, 64, 72, 128]))
    nseq = int(rng.integers(1, 7))
    lens_q = [int(x) for x in rng.integers(0, 200, nseq)]
    lens_k = [int(x) for x in rng.integers(0, 200, nseq)]
    kind = str(rng.choice(["full", "causal", "window"]))
    mask = {"full": {}, "causal": dict(causal=True),
            "window": dict(window_size=(int(rng.integers(-1, 50)), int(rng.integers(-1, 50))))}[kind]
    return dict(dtype=dtype, d=d, hkv=int(rng.choice([1, 2])), g=int(rng.choice([1, 2, 4])), lens_q=lens_q,
                lens_k=lens_k, mask=mask, scale=float(np.sqrt(rng.uniform(0.25, 2.0) / d)))


@pytest.mark.parametrize("i", range(VARLEN_CASES), ids=[f"varlen_{i}" for i in range(VARLEN_CASES)])
def test_random_varlen(i):
    from test_varlen_gpu import _draw, _run

    c = draw_varlen(i)
    print(f"fuzz varlen case {i}: {c}", flush=True)
    lq, lk = c["lens_q"], c["lens_k"]
    q, k, v, do, cu_q, cu_k = _draw(lq, lk, c["hkv"] * c["g"], c["hkv"], c["d"], c["dtype"], seed=i)
    kw = dict(c["mask"], scale=c["scale"])
    o, lse, dq, dk, dv = _run(q, k, v, do, cu_q, cu_k, max(max(lq), 1), max(max(lk), 1), **kw)
    okw = dict(causal=kw.get("causal", False), window=tuple(kw.get("window_size", (-1, -1))), scale=c["scale"])
    o_ref, lse_ref = oracle.attention_fwd_varlen(f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(), **okw)
    g_ref = oracle.attention_bwd_varlen(f64(do), f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(), **okw)
    tq, tk, tol = sum(lq), sum(lk), TOL[q.dtype]
    if tq:
        assert_close(lse[:, :tq], lse_ref[:, :tq], tol, "LSE")
    if c["dtype"] == "fp32":
        if tq:
            assert_close(o[:tq], o_ref[:tq], tol, "O")
            assert_close(dq[:tq], g_ref[0][:tq], 2 * tol, "dq")
        if tk:
            assert_close(dk[:tk], g_ref[1][:tk], 2 * tol, "dk")
            assert_close(dv[:tk], g_ref[2][:tk], 2 * tol, "dv")
        return
    # 16-bit: each sequence against the rounding model of that sequence.
    dt = DTYPE_NAME[q.dtype]
    cq, ck = cu_q.numpy(), cu_k.numpy()
    pw = dict(causal=okw["causal"], window=okw["window"], scale=okw["scale"])
    for s in range(len(lq)):
        a, b, c0, c1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if a == b:
            continue
        qs, ks, vs, dos = (f64(t)[None] for t in (q[a:b], k[c0:c1], v[c0:c1], do[a:b]))
        hold(f64(o[a:b])[None], o_ref[a:b][None], policy_fwd(qs, ks, vs, dt, **pw), dt, tol, f"O seq {s}")
        model = policy_grads(dos, qs, ks, vs, dt, **pw)
        hold(f64(dq[a:b])[None], g_ref[0][a:b][None], model[0], dt, 2 * tol, f"dq seq {s}")
        if c0 < c1:
            hold(f64(dk[c0:c1])[None], g_ref[1][c0:c1][None], model[1], dt, 2 * tol, f"dk seq {s}")
            hold(f64(dv[c0:c1])[None], g_ref[2][c0:c1][None], model[2], dt, 2 * tol, f"dv seq {s}")


def draw_kv(i):
    rng = np.random.default_rng(30_000 + i)
    dtype = str(rng.choice(["fp16", "bf16"]))
    d = int(rng.choice([8, 32, 64, 72, 128]))
    b = int(rng.integers(1, 4))
    nq = int(rng.integers(1, 9))
    cap = int(rng.integers(32, 400))
    lens = [int(x) for x in rng.integers(0, cap + 4, b)]  # some overflow the capacity
    kind = str(rng.choice(["full", "causal", "window"]))
    mask = {"full": {}, "causal": dict(causal=True),
            "window": dict(window_size=(int(rng.integers(-1, 120)), int(rng.integers(-1, 4))))}[kind]
    return dict(dtype=dtype, d=d, b=b, nq=nq, cap=cap, lens=lens, hkv=int(rng.choice([1, 2])),
                g=int(rng.choice([1, 2, 3, 4])), append=bool(rng.integers(0, 2)), splits=int(rng.choice([0, 1, 2, 5])),
                mask=mask, scale=float(np.sqrt(rng.uniform(0.25, 2.0) / d)))


@pytest.mark.parametrize("i", range(KV_CASES), ids=[f"kv_{i}" for i in range(KV_CASES)])
def test_random_kvcache(i):
    from test_kvcache_gpu import _draw, check_kv

    c = draw_kv(i)
    print(f"fuzz kvcache case {i}: {c}", flush=True)
    q, kc, vc, kn, vn = _draw(c["b"], c["nq"], c["hkv"] * c["g"], c["hkv"], c["d"], c["cap"], c["dtype"], seed=i)
    if not c["append"]:
        kn = vn = None
    check_kv(q, kc, vc, c["lens"], kn, vn, num_splits=c["splits"], **dict(c["mask"], scale=c["scale"]))
