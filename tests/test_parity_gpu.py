"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small cases span several tiles and ragged tails; every named workload runs at
its full size in the benchmark's launch configuration and is compared on
sampled heads that the oracle computes completely.
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
from exact_tiled_attention_07_amd.workloads import WORKLOADS, make_inputs, random_qkv  # noqa: E402
from gpu_util import TOL, assert_close, check_bwd, check_fwd, f64, gpu_bwd, gpu_fwd, max_err, record_errors  # noqa: E402,E501

DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
MASKS = [
    dict(),
    dict(causal=True),
    dict(window_size=(0, 0)),
    dict(window_size=(16, 0)),
    dict(window_size=(5, 3)),
    dict(causal=True, window_size=(40, -1)),
]
MASK_IDS = ["full", "causal", "self", "w16_0", "w5_3", "causal_w40"]


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# Small sweeps: sizes around the tile edges, all mask modes, MQA/GQA groups.
# ---------------------------------------------------------------------------
SIZES = [  # (B, N, Hq, Hkv)
    (1, 1, 2, 1), (2, 7, 4, 2), (1, 63, 2, 2), (1, 64, 8, 1), (2, 65, 4, 4),
    (1, 127, 8, 8), (1, 129, 4, 1), (1, 300, 32, 4),
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=MASK_IDS)
def test_fwd_sweep_mfma(dtype, d, mask):
    for i, (b, n, hq, hkv) in enumerate(SIZES):
        _note(f"fwd {dtype} d={d} {mask} B={b} N={n} Hq={hq} Hkv={hkv}")
        q, k, v, _ = random_qkv((b, n, hq, d), (b, n, hkv, d), dtype, seed=100 + i)
        check_fwd(q, k, v, **mask)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=MASK_IDS)
def test_bwd_sweep_mfma(dtype, d, mask):
    for i, (b, n, hq, hkv) in enumerate(SIZES):
        _note(f"bwd {dtype} d={d} {mask} B={b} N={n} Hq={hq} Hkv={hkv}")
        q, k, v, do = random_qkv((b, n, hq, d), (b, n, hkv, d), dtype, seed=200 + i)
        check_bwd(q, k, v, do, **mask)


@pytest.mark.parametrize("d", [4, 12, 64, 100, 128])
@pytest.mark.parametrize("mask", MASKS, ids=MASK_IDS)
def test_fp32_sweep(d, mask):
    for i, (b, n, hq, hkv) in enumerate(SIZES[:7]):
        _note(f"fp32 d={d} {mask} B={b} N={n} Hq={hq} Hkv={hkv}")
        q, k, v, do = random_qkv((b, n, hq, d), (b, n, hkv, d), "fp32", seed=300 + i)
        check_fwd(q, k, v, **mask)
        check_bwd(q, k, v, do, **mask)


# ---------------------------------------------------------------------------
# Unequal query/key lengths (queries aligned to the end of the keys), including
# rows that see no key at all.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("nq,nk", [(1, 300), (17, 200), (200, 17), (130, 1), (64, 129)])
@pytest.mark.parametrize("mask", [dict(), dict(causal=True), dict(window_size=(8, 2)),
                                  dict(causal=True, window_size=(3, -1))], ids=["full", "causal", "w8_2", "cw3"])
def test_unequal_lengths(dtype, nq, nk, mask):
    _note(f"unequal {dtype} Nq={nq} Nk={nk} {mask}")
    q, _, _, do = random_qkv((2, nq, 4, 64), (2, nq, 2, 64), dtype, seed=nq * 1000 + nk)
    _, k, v, _ = random_qkv((2, nk, 4, 64), (2, nk, 2, 64), dtype, seed=nq + 7 * nk)
    check_fwd(q, k, v, **mask)
    check_bwd(q, k, v, do, **mask)


@pytest.mark.parametrize("dtype,scales", [("fp32", (0.02, 0.3)), ("fp16", (0.02, 0.15)), ("bf16", (0.02, 0.15))])
def test_scale_parameter(dtype, scales):
    q, k, v, do = random_qkv((2, 100, 4, 128), (2, 100, 2, 128), dtype, seed=5)
    for s in scales:
        check_fwd(q, k, v, causal=True, scale=s)
        check_bwd(q, k, v, do, causal=True, scale=s)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.xfail(strict=True, reason="16-bit dS: the kernels round dS = P * (dP - D) to the input type before "
                                       "the dQ and dK products; at scale 0.3 (score std 3.4) that rounding alone "
                                       "puts dQ at about 1.3x the gradient bound")
def test_scale_parameter_large_16bit(dtype):
    # The forward meets its bound at this scale; the gradients do not.
    q, k, v, do = random_qkv((2, 100, 4, 128), (2, 100, 2, 128), dtype, seed=5)
    check_fwd(q, k, v, causal=True, scale=0.3)
    check_bwd(q, k, v, do, causal=True, scale=0.3)


# ---------------------------------------------------------------------------
# Empty and degenerate inputs.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_empty_inputs(dtype):
    dt = DT[dtype]
    dev = "cuda"
    q = torch.randn(0, 16, 2, 64, device=dev).to(dt)
    o, lse = fa.fwd(q, q, q)
    assert o.shape == q.shape and lse.shape == (0, 2, 16)
    q = torch.randn(2, 0, 2, 64, device=dev).to(dt)
    k = torch.randn(2, 10, 2, 64, device=dev).to(dt)
    o, lse = fa.fwd(q, k, k)
    assert o.numel() == 0
    dq, dk, dv = fa.bwd(q, q, k, k, o, lse)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)  # no queries: zero key gradients
    # no keys: every row sees nothing
    q = torch.randn(2, 5, 2, 64, device=dev).to(dt)
    k = torch.randn(2, 0, 2, 64, device=dev).to(dt)
    o, lse = fa.fwd(q, k, k, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    dq, dk, dv = fa.bwd(torch.randn_like(q), q, k, k, o, lse, causal=True)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


# ---------------------------------------------------------------------------
# Invariants that hold at any size.
# ---------------------------------------------------------------------------
def test_self_window_returns_values_exactly():
    q, k, v, _ = random_qkv((2, 333, 8, 128), (2, 333, 4, 128), "bf16", seed=11)
    o, lse = gpu_fwd(q, k, v, window_size=(0, 0))
    vv = v.cuda().repeat_interleave(2, dim=2)
    assert torch.equal(o, vv)


def test_zero_query_gives_mean_of_visible_values():
    q, k, v, _ = random_qkv((1, 257, 4, 64), (1, 257, 4, 64), "fp16", seed=12)
    q = torch.zeros_like(q)
    o, lse = gpu_fwd(q, k, v, causal=True)
    vf = f64(v)
    mean = np.cumsum(vf, axis=1) / np.arange(1, 258)[None, :, None, None]
    assert max_err(f64(o), mean) <= TOL[torch.float16]
    assert max_err(f64(lse), np.log(np.arange(1, 258))[None, None, :].repeat(4, 1)) <= 1e-5


def test_key_shift_invariance():
    q, k, v, _ = random_qkv((1, 500, 4, 128), (1, 500, 4, 128), "fp32", seed=13)
    u = torch.randn(128, generator=torch.Generator().manual_seed(3))
    o1, l1 = gpu_fwd(q, k, v, causal=True)
    o2, l2 = gpu_fwd(q, k + u, v, causal=True)
    shift = (q.double() @ u.double()).permute(0, 2, 1) / np.sqrt(128)
    assert max_err(f64(o2), f64(o1)) <= 2e-5
    assert max_err(f64(l2), f64(l1) + shift.numpy()) <= 2e-4


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_bitwise_repeatable(dtype):
    q, k, v, do = random_qkv((2, 1000, 8, 128), (2, 1000, 2, 128), dtype, seed=14)
    o1, l1 = gpu_fwd(q, k, v, causal=True)
    o2, l2 = gpu_fwd(q, k, v, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = gpu_bwd(do, q, k, v, o1, l1, causal=True)
    g2 = gpu_bwd(do, q, k, v, o1, l1, causal=True)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_bitwise_repeatable_bench_workload():
    # The benchmark workload at full size, four forward + backward passes: every
    # output equal to the first pass's bit for bit (no atomics, no data races on
    # the LDS buffers the tile loads rotate through).
    w = WORKLOADS["bf16_b2_hq32_hkv8_n8192_d128_causal"]
    q, k, v, do = (t.cuda() for t in make_inputs(w))
    ref = None
    for _ in range(4):
        o, lse = fa.fwd(q, k, v, causal=True)
        outs = (o, lse) + tuple(fa.bwd(do, q, k, v, o, lse, causal=True))
        torch.cuda.synchronize()
        if ref is None:
            ref = [t.clone() for t in outs]
            continue
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), ref, outs):
            assert torch.equal(a, b), name


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_backward_stages_equal_fa_bwd(dtype):
    # fa_bwd_stage PREPARE then DQ then DKDV (the two gradient stages in the
    # opposite order to fa_bwd's) gives fa_bwd's gradients bit for bit.
    q, k, v, do = (t.cuda() for t in random_qkv((2, 333, 8, 64), (2, 333, 4, 64), dtype, seed=17))
    o, lse = fa.fwd(q, k, v, causal=True)
    ref = fa.bwd(do, q, k, v, o, lse, causal=True)
    p = fa.make_params(q, k, v, o, causal=True)
    ws = torch.empty(fa.bwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)
    for st in (fa.FA_BWD_PREPARE, fa.FA_BWD_DQ, fa.FA_BWD_DKDV):
        fa.bwd(do, q, k, v, o, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws, stage=st)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)


def test_strided_packed_qkv_matches_contiguous():
    qkv = torch.randn(2, 200, 3, 8, 128, generator=torch.Generator().manual_seed(15)).to(torch.bfloat16).cuda()
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q.contiguous(), k.contiguous(), v.contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    do = torch.randn_like(o1)
    g1 = fa.bwd(do, q, k, v, o1, l1, causal=True)
    g2 = fa.bwd(do, q.contiguous(), k.contiguous(), v.contiguous(), o1, l1, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.contiguous(), b)


@pytest.mark.parametrize("which", ["kv", "q"])
def test_single_row_any_stride(which):
    # A tensor of one row along the sequence may carry any stride there, 0
    # included (an expanded view): the results equal those of contiguous copies.
    _note(f"single row, sequence stride 0: {which}")
    nq, nk = (70, 1) if which == "kv" else (1, 90)
    q, _, _, do = random_qkv((2, nq, 4, 128), (2, nq, 2, 128), "bf16", seed=31)
    _, k, v, _ = random_qkv((2, nk, 4, 128), (2, nk, 2, 128), "bf16", seed=32)
    q, k, v, do = (t.cuda() for t in (q, k, v, do))

    def zero_row_stride(t):
        return t.as_strided(t.shape, (t.stride(0), 0, t.stride(2), t.stride(3)))

    qs, ks, vs = (zero_row_stride(q), k, v) if which == "q" else (q, zero_row_stride(k), zero_row_stride(v))
    for mask in (dict(), dict(causal=True)):
        o1, l1 = fa.fwd(qs, ks, vs, **mask)
        o2, l2 = fa.fwd(q, k, v, **mask)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), mask
        g1 = fa.bwd(do, qs, ks, vs, o2, l2, **mask)
        g2 = fa.bwd(do, q, k, v, o2, l2, **mask)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a.contiguous(), b.contiguous()), mask


def test_autograd_wrapper_matches_bwd():
    q, k, v, do = (t.cuda() for t in random_qkv((1, 150, 4, 64), (1, 150, 2, 64), "fp16", seed=16))
    qr, kr, vr = (t.clone().requires_grad_() for t in (q, k, v))
    o = fa.attention(qr, kr, vr, causal=True)
    o.backward(do)
    o2, lse = fa.fwd(q, k, v, causal=True)
    g = fa.bwd(do, q, k, v, o2, lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for a, b in zip((qr.grad, kr.grad, vr.grad), g):
        assert torch.equal(a, b)


def test_native_library_is_loaded():
    q = torch.zeros(1, 8, 1, 64, device="cuda", dtype=torch.bfloat16)
    fa.fwd(q, q, q)
    maps = open("/proc/self/maps").read()
    assert fa.library_path() in maps


# ---------------------------------------------------------------------------
# The named workloads at full size, sampled heads against the oracle.
# ---------------------------------------------------------------------------
def _head_slices(w, q, k, v, do, b, g):
    """Inputs of one (batch, kv head) group: its G query heads and its K/V head."""
    G = w.nheads_q // w.nheads_kv
    sl = slice(g * G, (g + 1) * G)
    return (f64(q[b:b + 1, :, sl]), f64(k[b:b + 1, :, g:g + 1]), f64(v[b:b + 1, :, g:g + 1]),
            f64(do[b:b + 1, :, sl]), sl)


def _sample_rows(n):
    """Rows checked on every head at full size: the first, both sides of a
    256-query workgroup boundary, a row inside a diagonal tile in the middle,
    and the last."""
    return sorted({0, min(255, n - 1), min(256, n - 1), min(n // 2 + 77, n - 1), n - 1})


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(name):
    w = WORKLOADS[name]
    _note(f"workload {name}")
    q, k, v, do = make_inputs(w)
    kw = dict(causal=w.causal, window_size=w.window)
    o, lse = gpu_fwd(q, k, v, **kw)
    dq = dk = dv = None
    if w.backward:
        dq, dk, dv = gpu_bwd(do, q, k, v, o, lse, **kw)
    tol = TOL[DT[w.dtype]]
    ow = dict(causal=w.causal, window=w.window)
    small = w.batch * w.nheads_q * w.seqlen <= 16 * 1024 * 2
    # Whole (batch, kv head) groups: all of them for small workloads, else two on
    # different batch entries and XCDs (unit b * Hkv + g runs on XCD unit % 8).
    groups = [(b, g) for b in range(w.batch) for g in range(w.nheads_kv)] if small else \
        sorted({(w.batch - 1, w.nheads_kv - 1), (0, 0)})
    errors = {}
    for b, g in groups:
        qs, ks, vs, dos, sl = _head_slices(w, q, k, v, do, b, g)
        _note(f"  oracle group b={b} g={g}")
        o_ref, l_ref = oracle.attention_fwd(qs, ks, vs, **ow)
        info = {"o": assert_close(o[b:b + 1, :, sl], o_ref, tol, "O"),
                "lse": assert_close(lse[b:b + 1, sl], l_ref, tol, "LSE")}
        if w.backward:
            rq, rk, rv = oracle.attention_bwd(dos, qs, ks, vs, **ow)
            info["dq"] = assert_close(dq[b:b + 1, :, sl], rq, 2 * tol, "dQ")
            info["dk"] = assert_close(dk[b:b + 1, :, g:g + 1], rk, 2 * tol, "dK")
            info["dv"] = assert_close(dv[b:b + 1, :, g:g + 1], rv, 2 * tol, "dV")
        _note("  " + ", ".join(f"{n}: max-abs {e['raw']:.2e} at |ref| {e['raw_ref']:.3g}" for n, e in info.items()))
        for n, e in info.items():
            if n not in errors or e["raw"] > errors[n]["raw"]:
                errors[n] = e
    if not small:
        # Every (batch, query head) on sampled rows, one row at a time in the oracle.
        rows = _sample_rows(w.seqlen)
        qf, kf, vf = f64(q), f64(k), f64(v)
        o_got = f64(o)[:, rows].transpose(0, 2, 1, 3)  # (B, Hq, R, d)
        l_got = f64(lse)[:, :, rows]
        o_ref = np.empty_like(o_got)
        l_ref = np.empty_like(l_got)
        for b in range(w.batch):
            for h in range(w.nheads_q):
                o_ref[b, h], l_ref[b, h] = oracle.attention_fwd_rows(qf, kf, vf, b, h, rows, **ow)
        _note(f"  rows {rows} of all {w.batch * w.nheads_q} heads")
        for n, got, ref in (("o_rows", o_got, o_ref), ("lse_rows", l_got, l_ref)):
            e = assert_close(torch.from_numpy(got).to(DT[w.dtype] if n == "o_rows" else torch.float32), ref, tol, n)
            errors[n] = e
    record_errors(f"workload_{name}", errors)
    # Properties of the whole output (every head, not only the sampled ones).
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    if w.backward:
        assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
        # sum_j dK_j = 0 per (batch, kv head): rows of dS sum to zero.
        s = dk.double().sum(dim=1).abs().max().item()
        assert s <= 2 * tol * np.sqrt(w.seqlen), s
