"""GPU parity of attention against a KV cache (fa_fwd_kvcache) with the float64
oracle (oracle.kvcache_fwd): outputs and LSE to the O/LSE tolerance of the main
path, the cache contents after the in-place append bit for bit.

Cases cover single- and multi-token decode, chunked prefill, MQA/GQA packing
(more than 32 packed query rows, ragged), every mask mode, explicit and
automatic split counts, ragged / empty / full / overflowing cache lengths,
strided views, and every decode workload at full size in the launch
configuration the benchmark times.
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
from exact_tiled_attention_07_amd.workloads import DECODE_WORKLOADS, DTYPES, make_decode_inputs  # noqa: E402
from gpu_util import TOL, assert_close, f64  # noqa: E402

MASKS = [dict(), dict(causal=True), dict(window_size=(16, 0)), dict(causal=True, window_size=(40, -1)),
         dict(window_size=(5, 3))]
MASK_IDS = ["full", "causal", "w16_0", "causal_w40", "w5_3"]


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle_kw(kw):
    return dict(causal=kw.get("causal", False), window=tuple(kw.get("window_size", (-1, -1))),
                scale=kw.get("scale"))


def _draw(b, nq, hq, hkv, d, cap, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    dt = DTYPES[dtype]
    q = torch.randn((b, nq, hq, d), generator=g).to(dt)
    kc = torch.randn((b, cap, hkv, d), generator=g).to(dt)
    vc = torch.randn((b, cap, hkv, d), generator=g).to(dt)
    kn = torch.randn((b, nq, hkv, d), generator=g).to(dt)
    vn = torch.randn((b, nq, hkv, d), generator=g).to(dt)
    return q, kc, vc, kn, vn


def check_kv(q, kc, vc, lens, kn=None, vn=None, num_splits=0, tol_mult=1.0, **kw):
    """Runs the HIP path on device copies, the oracle on the CPU inputs, and
    compares O, LSE and both caches.  Returns the GPU (o, lse)."""
    qd, kcd, vcd = q.cuda(), kc.cuda(), vc.cuda()
    knd = kn.cuda() if kn is not None else None
    vnd = vn.cuda() if vn is not None else None
    lens_d = torch.as_tensor(lens, dtype=torch.int32).cuda()
    o, lse = fa.fwd_kvcache(qd, kcd, vcd, lens_d, knd, vnd, num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref, kc_ref, vc_ref = oracle.kvcache_fwd(
        f64(q), f64(kc), f64(vc), np.asarray(lens, dtype=np.int64), None if kn is None else f64(kn),
        None if vn is None else f64(vn), **_oracle_kw(kw))
    tol = TOL[q.dtype] * tol_mult
    assert_close(o, o_ref, tol, "O")
    assert_close(lse, lse_ref, tol, "LSE")
    assert np.array_equal(f64(kcd), kc_ref), "k_cache after the append differs"
    assert np.array_equal(f64(vcd), vc_ref), "v_cache after the append differs"
    return o, lse


# ---------------------------------------------------------------------------
# Small sweeps.
# ---------------------------------------------------------------------------
CASES = [
    # (B, Nq, Hq, Hkv, cap, lens)
    (1, 1, 1, 1, 32, [0]),
    (2, 1, 8, 2, 100, [37, 99]),            # second entry: append fills the cache exactly
    (3, 1, 32, 8, 300, [299, 1, 150]),
    (2, 2, 4, 4, 64, [31, 62]),
    (2, 4, 16, 2, 257, [200, 9]),           # 8 x 4 = 32 packed rows
    (1, 5, 12, 2, 130, [64]),               # 6 x 5 = 30 packed rows
    (2, 20, 8, 2, 200, [0, 100]),           # 4 x 20 = 80 packed rows: three row blocks, ragged
    (1, 64, 4, 1, 129, [65]),               # chunk of 64 queries
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=MASK_IDS)
def test_kvcache_sweep(dtype, d, mask):
    for ci, (b, nq, hq, hkv, cap, lens) in enumerate(CASES):
        for splits in (0, 1, 3):
            _note(f"kvcache {dtype} d={d} {mask} B={b} Nq={nq} Hq={hq} Hkv={hkv} cap={cap} lens={lens} "
                  f"splits={splits}")
            q, kc, vc, kn, vn = _draw(b, nq, hq, hkv, d, cap, dtype, seed=400 + 10 * ci + splits)
            check_kv(q, kc, vc, lens, kn, vn, num_splits=splits, **mask)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("mask", MASKS[:2], ids=MASK_IDS[:2])
def test_kvcache_without_append(dtype, mask):
    for ci, (b, nq, hq, hkv, cap, lens) in enumerate(CASES):
        _note(f"kvcache no-append {dtype} {mask} B={b} Nq={nq} cap={cap} lens={lens}")
        q, kc, vc, _, _ = _draw(b, nq, hq, hkv, 128, cap, dtype, seed=500 + ci)
        check_kv(q, kc, vc, lens, **mask)


def test_kvcache_lengths_are_clamped_and_overflow_is_dropped():
    # Negative length -> 0; length past the capacity -> capacity (nothing
    # appended, all rows visible); L + Nq past the capacity -> only the rows
    # that fit are written.
    q, kc, vc, kn, vn = _draw(4, 6, 4, 2, 64, 70, "bf16", seed=7)
    for mask in (dict(), dict(causal=True)):
        check_kv(q, kc, vc, [-5, 1000, 67, 70], kn, vn, **mask)
        check_kv(q, kc, vc, [-5, 1000, 67, 70], **mask)


def test_kvcache_empty_cache_rows_see_nothing():
    # No valid rows and nothing appended: O = 0, LSE = -inf everywhere.
    q, kc, vc, _, _ = _draw(2, 3, 4, 2, 128, 96, "fp16", seed=8)
    o, lse = check_kv(q, kc, vc, [0, 0], causal=True)
    assert torch.count_nonzero(o).item() == 0
    assert torch.isneginf(lse).all()
    # Zero capacity with an append: still nothing to attend to.
    q, kc, vc, kn, vn = _draw(2, 3, 4, 2, 128, 0, "fp16", seed=9)
    o, lse = check_kv(q, kc, vc, [0, 0], kn, vn)
    assert torch.isneginf(lse).all()


def test_kvcache_empty_problems():
    dev = "cuda"
    q = torch.zeros(0, 1, 4, 128, dtype=torch.bfloat16, device=dev)
    c = torch.zeros(0, 64, 2, 128, dtype=torch.bfloat16, device=dev)
    o, lse = fa.fwd_kvcache(q, c, c, torch.zeros(0, dtype=torch.int32, device=dev))
    assert o.shape == q.shape and lse.shape == (0, 4, 1)
    q = torch.zeros(2, 0, 4, 128, dtype=torch.bfloat16, device=dev)
    c = torch.zeros(2, 64, 2, 128, dtype=torch.bfloat16, device=dev)
    o, lse = fa.fwd_kvcache(q, c, c, torch.zeros(2, dtype=torch.int32, device=dev))
    assert o.shape == q.shape and lse.shape == (2, 4, 0)
    torch.cuda.synchronize()


def test_kvcache_strided_views():
    # q is a head slice of a wider tensor; the caches are the K and V halves of
    # one packed (B, cap, 2 * Hkv, d) buffer; new rows come from a packed
    # (B, Nq, 2 * Hkv, d) tensor; out is a strided view too.
    g = torch.Generator("cpu").manual_seed(11)
    b, nq, hq, hkv, d, cap = 2, 3, 8, 2, 128, 150
    qw = torch.randn((b, nq, 2 * hq, d), generator=g).to(torch.bfloat16)
    kvc = torch.randn((b, cap, 2 * hkv, d), generator=g).to(torch.bfloat16)
    kvn = torch.randn((b, nq, 2 * hkv, d), generator=g).to(torch.bfloat16)
    lens = [40, 147]
    qd, kvcd, kvnd = qw.cuda(), kvc.cuda(), kvn.cuda()
    q = qd[:, :, hq:]
    kc, vc = kvcd[:, :, :hkv], kvcd[:, :, hkv:]
    kn, vn = kvnd[:, :, :hkv], kvnd[:, :, hkv:]
    outw = torch.zeros((b, nq, 2 * hq, d), dtype=torch.bfloat16, device="cuda")
    out = outw[:, :, :hq]
    o, lse = fa.fwd_kvcache(q, kc, vc, torch.tensor(lens, dtype=torch.int32, device="cuda"), kn, vn,
                            causal=True, out=out)
    torch.cuda.synchronize()
    o_ref, lse_ref, kc_ref, vc_ref = oracle.kvcache_fwd(
        f64(qw[:, :, hq:]), f64(kvc[:, :, :hkv]), f64(kvc[:, :, hkv:]), np.array(lens), f64(kvn[:, :, :hkv]),
        f64(kvn[:, :, hkv:]), causal=True)
    assert_close(out, o_ref, TOL[torch.bfloat16], "O")
    assert_close(lse, lse_ref, TOL[torch.bfloat16], "LSE")
    assert torch.count_nonzero(outw[:, :, hq:]).item() == 0, "write outside the output view"
    assert np.array_equal(f64(kvcd[:, :, :hkv]), kc_ref) and np.array_equal(f64(kvcd[:, :, hkv:]), vc_ref)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_token_by_token_decode_matches_full_causal_attention(dtype):
    # Prefill with the main forward is not involved: the cache starts with 50
    # valid rows and 12 tokens are decoded one by one, the lengths advanced on
    # the device.  Every step's output is the matching row of one causal
    # attention over the whole 62-token sequence.
    g = torch.Generator("cpu").manual_seed(12)
    b, n0, steps, hq, hkv, d, cap = 2, 50, 12, 8, 2, 128, 64
    dt = DTYPES[dtype]
    q_all = torch.randn((b, n0 + steps, hq, d), generator=g).to(dt)
    k_all = torch.randn((b, n0 + steps, hkv, d), generator=g).to(dt)
    v_all = torch.randn((b, n0 + steps, hkv, d), generator=g).to(dt)
    kc = torch.zeros((b, cap, hkv, d), dtype=dt, device="cuda")
    vc = torch.zeros((b, cap, hkv, d), dtype=dt, device="cuda")
    kc[:, :n0] = k_all[:, :n0].cuda()
    vc[:, :n0] = v_all[:, :n0].cuda()
    lens = torch.full((b,), n0, dtype=torch.int32, device="cuda")
    o_ref, lse_ref = oracle.attention_fwd(f64(q_all), f64(k_all), f64(v_all), causal=True)
    for t in range(n0, n0 + steps):
        o, lse = fa.fwd_kvcache(q_all[:, t:t + 1].cuda(), kc, vc, lens, k_all[:, t:t + 1].cuda(),
                                v_all[:, t:t + 1].cuda(), causal=True)
        lens += 1
        torch.cuda.synchronize()
        assert_close(o, o_ref[:, t:t + 1], TOL[dt], f"O step {t}")
        assert_close(lse, lse_ref[:, :, t:t + 1], TOL[dt], f"LSE step {t}")
    assert torch.equal(kc[:, :n0 + steps].cpu(), k_all) and torch.equal(vc[:, :n0 + steps].cpu(), v_all)


def test_kvcache_is_deterministic_and_split_count_changes_only_rounding():
    q, kc, vc, _, _ = _draw(2, 1, 32, 8, 128, 4000, "bf16", seed=13)
    qd, kcd, vcd = q.cuda(), kc.cuda(), vc.cuda()
    lens = torch.tensor([3999, 2500], dtype=torch.int32, device="cuda")
    o1, l1 = fa.fwd_kvcache(qd, kcd, vcd, lens)
    o2, l2 = fa.fwd_kvcache(qd, kcd, vcd, lens)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref, _, _ = oracle.kvcache_fwd(f64(q), f64(kc), f64(vc), np.array([3999, 2500]))
    for splits in (1, 2, 7, 32, 125):
        o, lse = fa.fwd_kvcache(qd, kcd, vcd, lens, num_splits=splits)
        torch.cuda.synchronize()
        assert_close(o, o_ref, TOL[torch.bfloat16], f"O splits={splits}")
        assert_close(lse, lse_ref, TOL[torch.bfloat16], f"LSE splits={splits}")


def test_kvcache_caller_workspace():
    q, kc, vc, kn, vn = _draw(2, 2, 8, 2, 64, 300, "fp16", seed=14)
    p = fa.make_kv_params(q, kc, vc, q, kn, vn, causal=True)
    need = fa.kvcache_workspace_size(p)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # stale contents must not matter
    qd, kcd, vcd = q.cuda(), kc.cuda(), vc.cuda()
    o, lse = fa.fwd_kvcache(qd, kcd, vcd, torch.tensor([10, 290], dtype=torch.int32, device="cuda"), kn.cuda(),
                            vn.cuda(), causal=True, workspace=ws)
    torch.cuda.synchronize()
    o_ref, lse_ref, _, _ = oracle.kvcache_fwd(f64(q), f64(kc), f64(vc), np.array([10, 290]), f64(kn), f64(vn),
                                              causal=True)
    assert_close(o, o_ref, TOL[torch.float16], "O")
    assert_close(lse, lse_ref, TOL[torch.float16], "LSE")
    with pytest.raises(fa.FaError, match="workspace"):
        fa.fwd_kvcache(qd, kcd, vcd, torch.tensor([10, 290], dtype=torch.int32, device="cuda"), kn.cuda(),
                       vn.cuda(), causal=True, workspace=ws[:need - 256])


def test_kvcache_rejects_fp32_and_odd_head_sizes():
    c = torch.zeros(1, 64, 1, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError, match="UNSUPPORTED"):
        fa.fwd_kvcache(torch.zeros(1, 1, 1, 64, device="cuda"), c, c, torch.zeros(1, dtype=torch.int32,
                                                                                    device="cuda"))
    for d in (136, 256, 100):  # above 128, or not a multiple of 8
        c = torch.zeros(1, 64, 1, d, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(fa.FaError, match="UNSUPPORTED"):
            fa.fwd_kvcache(torch.zeros(1, 1, 1, d, dtype=torch.bfloat16, device="cuda"), c, c,
                           torch.zeros(1, dtype=torch.int32, device="cuda"))


# ---------------------------------------------------------------------------
# Every decode workload at full size, automatic split count (the benchmark's
# launch configuration); the oracle runs per batch entry.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_decode_workload_full_size(name):
    w = DECODE_WORKLOADS[name]
    _note(f"decode workload {name}")
    q, kc, vc, kn, vn, lens = make_decode_inputs(w)
    kw = dict(causal=w.causal, window_size=w.window)
    qd, kcd, vcd, knd, vnd, lensd = (t.cuda() for t in (q, kc, vc, kn, vn, lens))
    o, lse = fa.fwd_kvcache(qd, kcd, vcd, lensd, knd, vnd, **kw)
    torch.cuda.synchronize()
    tol = TOL[DTYPES[w.dtype]]
    for b in range(w.batch):
        lb = lens[b:b + 1].numpy().astype(np.int64)
        o_ref, lse_ref, kc_ref, vc_ref = oracle.kvcache_fwd(
            f64(q[b:b + 1]), f64(kc[b:b + 1]), f64(vc[b:b + 1]), lb, f64(kn[b:b + 1]), f64(vn[b:b + 1]),
            **_oracle_kw(kw))
        assert_close(o[b:b + 1], o_ref, tol, f"O entry {b}")
        assert_close(lse[b:b + 1], lse_ref, tol, f"LSE entry {b}")
        lo, hi = int(lens[b]), int(lens[b]) + w.nq
        assert np.array_equal(f64(kcd[b, lo:hi]), kc_ref[0, lo:hi])
        assert np.array_equal(f64(vcd[b, lo:hi]), vc_ref[0, lo:hi])
    # Rows outside the appended range are untouched.
    mask = torch.ones(kc.shape[:2], dtype=torch.bool)
    for b in range(w.batch):
        mask[b, int(lens[b]):int(lens[b]) + w.nq] = False
    assert torch.equal(kcd.cpu()[mask], kc[mask]) and torch.equal(vcd.cpu()[mask], vc[mask])


# ---------------------------------------------------------------------------
# Paged caches (fa_fwd_kvcache_paged).
# ---------------------------------------------------------------------------
def _paged_from(kc, vc, ps, rng, spare=3):
    """Scatter contiguous (B, cap, H, d) caches into a shuffled page pool with
    spare pages; returns (k_pages, v_pages, table)."""
    nb, cap = kc.shape[:2]
    per = cap // ps
    n_pages = nb * per + spare
    perm = torch.from_numpy(rng.permutation(n_pages)).long()
    table = perm[:nb * per].reshape(nb, per).to(torch.int32)
    g = torch.Generator("cpu").manual_seed(int(rng.integers(1 << 31)))
    kp = torch.randn((n_pages, ps) + tuple(kc.shape[2:]), generator=g).to(kc.dtype)
    vp = torch.randn((n_pages, ps) + tuple(kc.shape[2:]), generator=g).to(kc.dtype)
    for b in range(nb):
        for p in range(per):
            kp[table[b, p]] = kc[b, p * ps:(p + 1) * ps]
            vp[table[b, p]] = vc[b, p * ps:(p + 1) * ps]
    return kp, vp, table


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("ps", [32, 64, 256])
@pytest.mark.parametrize("mask", [dict(causal=True), dict(window_size=(40, 0)), dict()], ids=["causal", "w40", "full"])
def test_paged_matches_oracle(dtype, d, ps, mask):
    rng = np.random.default_rng(ps + d)
    for append in (True, False):
        b, nq, hq, hkv, cap = 3, 2, 8, 2, 4 * 256
        q, kc, vc, kn, vn = _draw(b, nq, hq, hkv, d, cap, dtype, seed=900 + ps)
        lens = [cap - 1, 37, 600]  # the first entry overflows when appending
        kp, vp, table = _paged_from(kc, vc, ps, rng)
        _note(f"paged {dtype} d={d} ps={ps} {mask} append={append}")
        kpd, vpd = kp.cuda(), vp.cuda()
        o, lse = fa.fwd_kvcache_paged(q.cuda(), kpd, vpd, torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                      table.cuda(), kn.cuda() if append else None, vn.cuda() if append else None,
                                      **mask)
        torch.cuda.synchronize()
        o_ref, lse_ref, kp_ref, vp_ref = oracle.kvcache_fwd_paged(
            f64(q), f64(kp), f64(vp), np.array(lens), table.numpy(), f64(kn) if append else None,
            f64(vn) if append else None, causal=mask.get("causal", False),
            window=tuple(mask.get("window_size", (-1, -1))))
        assert_close(o, o_ref, TOL[q.dtype], "O")
        assert_close(lse, lse_ref, TOL[q.dtype], "LSE")
        assert np.array_equal(f64(kpd), kp_ref) and np.array_equal(f64(vpd), vp_ref), "pages after the append"


def test_paged_equals_contiguous_bitwise_full_size():
    # The benchmark's decode workload with its cache cut into 256-row pages in
    # a shuffled pool: the same tiles in the same order, so the same bits.
    w = DECODE_WORKLOADS["bf16_decode_b8_hq32_hkv8_d128_cap16384"]
    q, kc, vc, kn, vn, lens = make_decode_inputs(w)
    kp, vp, table = _paged_from(kc.contiguous(), vc.contiguous(), 256, np.random.default_rng(5))
    qd, knd, vnd, lensd = q.cuda(), kn.cuda(), vn.cuda(), lens.cuda()
    kcd, vcd = kc.cuda(), vc.cuda()
    o1, l1 = fa.fwd_kvcache(qd, kcd, vcd, lensd, knd, vnd, causal=True)
    kpd, vpd = kp.cuda(), vp.cuda()
    o2, l2 = fa.fwd_kvcache_paged(qd, kpd, vpd, lensd, table.cuda(), knd, vnd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for b in range(w.batch):
        r = int(lens[b])
        assert torch.equal(kpd[int(table[b, r // 256]), r % 256].cpu(), kn[b, 0])
        assert torch.equal(vpd[int(table[b, r // 256]), r % 256].cpu(), vn[b, 0])
