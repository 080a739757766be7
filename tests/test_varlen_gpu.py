"""GPU parity of packed variable-length batches (fa_fwd_varlen / fa_bwd_varlen)
and of packed q/k/v, through the C ABI.

* small ragged batches against the float64 oracle (oracle.attention_*_varlen),
  every dtype, head size and mask mode, zero-length sequences included;
* rows outside every sequence are never written;
* each sequence of a packed batch is bit for bit what fa_fwd / fa_bwd give for
  that sequence alone (same kernels, same tiles), also at full size, where the
  fixed-length path is itself checked against the oracle;
* packed q/k/v (strided views of one tensor) give the separate-tensor results
  bit for bit, gradients written into one packed tensor.
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
from exact_tiled_attention_07_amd.workloads import DTYPES  # noqa: E402
from gpu_util import TOL, assert_close, f64  # noqa: E402

MASKS = [dict(), dict(causal=True), dict(window_size=(16, 0)), dict(causal=True, window_size=(40, -1)),
         dict(window_size=(5, 3))]
MASK_IDS = ["full", "causal", "w16_0", "causal_w40", "w5_3"]
SENTINEL = 7.0


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _okw(kw):
    return dict(causal=kw.get("causal", False), window=tuple(kw.get("window_size", (-1, -1))),
                scale=kw.get("scale"))


def _draw(lens_q, lens_k, hq, hkv, d, dtype, seed, extra=0):
    g = torch.Generator("cpu").manual_seed(seed)
    dt = DTYPES[dtype]
    tq, tk = sum(lens_q) + extra, sum(lens_k) + extra
    q = torch.randn((tq, hq, d), generator=g).to(dt)
    k = torch.randn((tk, hkv, d), generator=g).to(dt)
    v = torch.randn((tk, hkv, d), generator=g).to(dt)
    do = torch.randn((tq, hq, d), generator=g).to(dt)
    cu_q = torch.tensor([0] + list(np.cumsum(lens_q)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(lens_k)), dtype=torch.int32)
    return q, k, v, do, cu_q, cu_k


def _run(q, k, v, do, cu_q, cu_k, max_q, max_k, **kw):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    cq, ck = cu_q.cuda(), cu_k.cuda()
    out = torch.full_like(qd, SENTINEL)
    o, lse = fa.fwd_varlen(qd, kd, vd, cq, ck, max_q, max_k, out=out, **kw)
    dq = torch.full_like(qd, SENTINEL)
    dk = torch.full_like(kd, SENTINEL)
    dv = torch.full_like(vd, SENTINEL)
    fa.bwd_varlen(dod, qd, kd, vd, o, lse, cq, ck, max_q, max_k, dq=dq, dk=dk, dv=dv, **kw)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


CASES = [
    # (lens_q, lens_k)
    ([64, 64, 64], [64, 64, 64]),
    ([1, 37, 128, 129, 5], [1, 37, 128, 129, 5]),
    ([300, 0, 17, 64], [300, 12, 0, 200]),      # a sequence without keys and one without queries
    ([1, 1, 1, 1], [257, 31, 1, 100]),           # decode-like: one query per sequence
    ([200, 17], [17, 200]),
]


@pytest.mark.parametrize("dtype,d", [("fp16", 64), ("bf16", 128), ("fp16", 128), ("bf16", 64), ("fp32", 64),
                                     ("fp32", 100)])
@pytest.mark.parametrize("mask", MASKS, ids=MASK_IDS)
def test_varlen_sweep(dtype, d, mask):
    for ci, (lq, lk) in enumerate(CASES):
        _note(f"varlen {dtype} d={d} {mask} lens_q={lq} lens_k={lk}")
        q, k, v, do, cu_q, cu_k = _draw(lq, lk, 4, 2, d, dtype, seed=600 + ci, extra=3)
        o, lse, dq, dk, dv = _run(q, k, v, do, cu_q, cu_k, max(lq), max(lk), **mask)
        o_ref, lse_ref = oracle.attention_fwd_varlen(f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(),
                                                     **_okw(mask))
        g_ref = oracle.attention_bwd_varlen(f64(do), f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(),
                                            **_okw(mask))
        tq, tk = sum(lq), sum(lk)
        tol = TOL[q.dtype]
        assert_close(o[:tq], o_ref[:tq], tol, "O")
        assert_close(lse[:, :tq], lse_ref[:, :tq], tol, "LSE")
        assert_close(dq[:tq], g_ref[0][:tq], 2 * tol, "dq")
        assert_close(dk[:tk], g_ref[1][:tk], 2 * tol, "dk")
        assert_close(dv[:tk], g_ref[2][:tk], 2 * tol, "dv")
        # The three packed rows after the last sequence are never written.
        for name, t in (("o", o[tq:]), ("dq", dq[tq:]), ("dk", dk[tk:]), ("dv", dv[tk:])):
            assert bool((t == SENTINEL).all()), f"{name} written outside every sequence"


# Packed causal batches whose (sequence, kv head) count is a multiple of 8 and
# at most 512: the dK/dV kernel hands each workgroup the next-heaviest key tile
# of its XCD's share (longest first), so every key tile of every sequence,
# empty ones included, must still be visited exactly once.
LPT_CASES = [
    # (lens_q, lens_k, hq, hkv)
    ([300, 0, 17, 129, 1, 64, 0, 200], [300, 12, 0, 129, 257, 64, 40, 17], 32, 8),
    ([513, 1, 64, 1000], [513, 1, 64, 1000], 16, 8),
    ([5, 1] * 32, [70, 1] * 32, 8, 8),                 # 64 sequences x 8 kv heads: 512 units
    ([0, 90, 33, 0], [129, 90, 0, 0], 8, 2),           # Hkv 2, 4 sequences: 8 units
]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
def test_varlen_causal_longest_first_key_tiles(dtype, d):
    for ci, (lq, lk, hq, hkv) in enumerate(LPT_CASES):
        assert (len(lq) * hkv) % 8 == 0 and len(lq) * hkv <= 512
        _note(f"varlen longest-first {dtype} d={d} hq={hq} hkv={hkv} lens_q={lq} lens_k={lk}")
        q, k, v, do, cu_q, cu_k = _draw(lq, lk, hq, hkv, d, dtype, seed=900 + ci, extra=2)
        o, lse, dq, dk, dv = _run(q, k, v, do, cu_q, cu_k, max(lq), max(lk), causal=True)
        o_ref, lse_ref = oracle.attention_fwd_varlen(f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(),
                                                     causal=True)
        g_ref = oracle.attention_bwd_varlen(f64(do), f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(),
                                            causal=True)
        tq, tk = sum(lq), sum(lk)
        tol = TOL[q.dtype]
        assert_close(o[:tq], o_ref[:tq], tol, "O")
        assert_close(lse[:, :tq], lse_ref[:, :tq], tol, "LSE")
        assert_close(dq[:tq], g_ref[0][:tq], 2 * tol, "dq")
        assert_close(dk[:tk], g_ref[1][:tk], 2 * tol, "dk")
        assert_close(dv[:tk], g_ref[2][:tk], 2 * tol, "dv")
        for b in range(len(lq)):
            k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
            if lq[b] == 0 and k1 > k0:  # keys that no query sees get zero gradients
                assert bool((dk[k0:k1] == 0).all()) and bool((dv[k0:k1] == 0).all()), b
        for name, t in (("o", o[tq:]), ("dq", dq[tq:]), ("dk", dk[tk:]), ("dv", dv[tk:])):
            assert bool((t == SENTINEL).all()), f"{name} written outside every sequence"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_varlen_sequences_equal_fixed_length_calls_bitwise(dtype):
    lq = [130, 1, 64, 257, 33]
    lk = [130, 300, 64, 257, 2]
    d = 128 if dtype == "bf16" else 64
    q, k, v, do, cu_q, cu_k = _draw(lq, lk, 8, 2, d, dtype, seed=7)
    for mask in (dict(causal=True), dict(window_size=(20, 4))):
        o, lse, dq, dk, dv = _run(q, k, v, do, cu_q, cu_k, max(lq), max(lk), **mask)
        for b in range(len(lq)):
            q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
            qs, ks, vs, dos = (t.cuda()[None] for t in (q[q0:q1], k[k0:k1], v[k0:k1], do[q0:q1]))
            ob, lb = fa.fwd(qs, ks, vs, **mask)
            gb = fa.bwd(dos, qs, ks, vs, ob, lb, **mask)
            torch.cuda.synchronize()
            assert torch.equal(o[q0:q1], ob[0]) and torch.equal(lse[:, q0:q1], lb[0]), b
            assert torch.equal(dq[q0:q1], gb[0][0]), b
            assert torch.equal(dk[k0:k1], gb[1][0]) and torch.equal(dv[k0:k1], gb[2][0]), b


def test_varlen_full_size_ragged_batch():
    # 16384 packed tokens of the benchmark's head shape (bf16, Hq=32, Hkv=8,
    # d=128, causal) in sequences of 8192 down to 256: each sequence is bit
    # for bit the fixed-length call on it, and sampled rows match the oracle.
    lq = [8192, 4096, 2048, 1024, 512, 256, 256]
    q, k, v, do, cu_q, cu_k = _draw(lq, lq, 32, 8, 128, "bf16", seed=1004)
    o, lse, dq, dk, dv = _run(q, k, v, do, cu_q, cu_k, max(lq), max(lq), causal=True)
    for b in (0, 3, 6):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        qs, ks, vs, dos = (t.cuda()[None] for t in (q[q0:q1], k[q0:q1], v[q0:q1], do[q0:q1]))
        ob, lb = fa.fwd(qs, ks, vs, causal=True)
        gb = fa.bwd(dos, qs, ks, vs, ob, lb, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[q0:q1], ob[0]) and torch.equal(lse[:, q0:q1], lb[0]), b
        assert torch.equal(dq[q0:q1], gb[0][0]) and torch.equal(dk[q0:q1], gb[1][0]), b
        assert torch.equal(dv[q0:q1], gb[2][0]), b
        rows = np.unique(np.linspace(0, q1 - q0 - 1, 9).astype(np.int64))
        qb, kb, vb = f64(q[None, q0:q1]), f64(k[None, q0:q1]), f64(v[None, q0:q1])
        for h in (0, 31):
            o_ref, l_ref = oracle.attention_fwd_rows(qb, kb, vb, 0, h, rows, causal=True)
            assert_close(o[q0:q1][rows, h], o_ref, TOL[torch.bfloat16], f"O seq {b} head {h}")
            assert_close(lse[h, q0:q1][rows], l_ref, TOL[torch.bfloat16], f"LSE seq {b} head {h}")


def test_varlen_autograd_wrapper():
    lq = [50, 3, 120]
    q, k, v, do, cu_q, cu_k = _draw(lq, lq, 4, 2, 64, "fp16", seed=8)
    qd, kd, vd = (t.cuda().requires_grad_() for t in (q, k, v))
    o = fa.attention_varlen(qd, kd, vd, cu_q.cuda(), cu_k.cuda(), max(lq), max(lq), causal=True)
    o.backward(do.cuda())
    o2, lse2, dq, dk, dv = _run(q, k, v, do, cu_q, cu_k, max(lq), max(lq), causal=True)
    assert torch.equal(o.detach(), o2)
    assert torch.equal(qd.grad, dq) and torch.equal(kd.grad, dk) and torch.equal(vd.grad, dv)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_qkvpacked_equals_separate_tensors_bitwise(dtype):
    g = torch.Generator("cpu").manual_seed(9)
    d = 128 if dtype == "bf16" else 64
    qkv = torch.randn((2, 200, 3, 8, d), generator=g).to(DTYPES[dtype]).cuda()
    do = torch.randn((2, 200, 8, d), generator=g).to(DTYPES[dtype]).cuda()
    o_p, lse_p = fa.fwd_qkvpacked(qkv, causal=True)
    q, k, v = (qkv[:, :, i].contiguous() for i in range(3))
    o_s, lse_s = fa.fwd(q, k, v, causal=True)
    assert torch.equal(o_p, o_s) and torch.equal(lse_p, lse_s)
    x = qkv.clone().requires_grad_()
    fa.attention_qkvpacked(x, causal=True).backward(do)
    dq, dk, dv = fa.bwd(do, q, k, v, o_s, lse_s, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(x.grad[:, :, 0], dq) and torch.equal(x.grad[:, :, 1], dk) and torch.equal(x.grad[:, :, 2], dv)
    o_ref, _ = oracle.attention_fwd(f64(q), f64(k), f64(v), causal=True)
    assert_close(o_p, o_ref, TOL[DTYPES[dtype]], "O")


def test_varlen_empty_and_rejected_inputs():
    dev = "cuda"
    q = torch.zeros(0, 4, 64, dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(1, dtype=torch.int32, device=dev)
    o, lse = fa.fwd_varlen(q, q[:, :2], q[:, :2], cu, cu, 0, 0)
    assert o.shape == q.shape and lse.shape == (4, 0)
    with pytest.raises(ValueError):
        fa.fwd_varlen(q, q[:, :2], q[:, :2], cu.to(torch.int64), cu, 0, 0)
    torch.cuda.synchronize()
