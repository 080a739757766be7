#!/usr/bin/env python3
"""Throughput of exact tiled attention (forward + backward) on one MI355X.

A step is one pass of the whole path -- fa_fwd then fa_bwd -- over the bf16
GQA causal workload B=2, N=8192, Hq=32, Hkv=8, d=128 with synthetic inputs
already resident in HBM.  Prints ONE JSON line (see --help).

Algorithmic FLOP: forward 4*B*Hq*N^2*d halved for causal, backward 2.5x the
forward (five products per visible score pair instead of two).

Beside the step, the same line carries a "decode" object: fa_fwd_kvcache
(in-place append + attention against a ragged KV cache) on the bf16 decode
workload B=8, one new token, Hq=32, Hkv=8, d=128, capacity 16384, timed per
call with events and priced against HBM bandwidth (it reads the cache once);
a "next_rows" object (packed variable-length batch, score modifiers); and a
"configs" object: fa_fwd and fa_bwd timed on their own on every named
workload at full size (median of 5 runs of at least --config-calls calls and
about 2 ms of work each); and a
"memory" object: the peak device memory of one forward + backward beyond the
inputs, against standard attention that keeps the N x N matrices; and a
"gemm_reference" object: the vendor library's bf16 GEMM rate on the same chip,
the dense matrix-core throughput it sustains under load.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s at 1 GPU (bf16, d=128, N=8K causal); % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published figure
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample (whole heads are added until it is reached)")
    ap.add_argument("--decode-calls", type=int, default=200, help="timed fa_fwd_kvcache calls (0: skip)")
    ap.add_argument("--next-rows-steps", type=int, default=10,
                    help="timed steps of the packed-batch and score-modifier legs (0: skip)")
    ap.add_argument("--config-calls", type=int, default=10,
                    help="minimum timed calls per repeat (5 repeats of at least 2 ms) of each named workload's "
                         "fwd and bwd (0: skip)")
    ap.add_argument("--no-memory", action="store_true", help="skip the peak-memory comparison")
    ap.add_argument("--no-gemm", action="store_true", help="skip the vendor bf16 GEMM reference rate")
    ap.add_argument("--copy-probe", action="store_true",
                    help="instead of the benchmark, run a plain device copy of 512 MiB (read 512 MiB, "
                         "write 512 MiB) 5 times: the known-size reference for HBM byte counters")
    return ap.parse_args()


def copy_probe():
    import torch
    n = 512 << 20
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                      "copy_GBps": round(2 * n / dt / 1e9, 1)}), flush=True)


def visible_pairs(n, causal, window):
    """Score pairs per (batch, head) by the counting convention of the metric:
    N^2/2 for a causal mask, N^2 without one, the exact count for a window."""
    wl, wr = window
    if wl < 0 and wr < 0:
        return n * n / 2 if causal else float(n * n)
    total = 0
    for i in range(n):
        lo = 0 if wl < 0 else max(0, i - wl)
        hi = i if causal else (n - 1 if wr < 0 else min(n - 1, i + wr))
        if causal and wr >= 0:
            hi = min(hi, i + wr)
        total += max(0, hi - lo + 1)
    return float(total)


def flops(w):
    fwd = 4.0 * w.batch * w.nheads_q * w.headdim * visible_pairs(w.seqlen, w.causal, w.window)
    return fwd, 2.5 * fwd


# Counter-derived figures per launch of the attention kernels on the bench
# workload, from rocprofv3 --pmc runs of "python3 bench.py --steps 2 --warmup 1
# --no-cpu-baseline --decode-calls 0 --next-rows-steps 0 --config-calls 0"
# (profiles/attention_kernels_bf16_b2_hq32_hkv8_n8192_d128_causal_counters.txt):
#   mfma_busy  SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8), the
#              share of the cycles the kernel ran at that its matrix cores were busy
#   traffic    HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled
#              by what the same counter needs to read 512 MiB for the plain copy of
#              "python3 bench.py --copy-probe"
# They describe the kernels built from the sources whose SHA-256 is recorded
# here and are reported as null for any other source.
COUNTERS = {
    "sources_sha256": "0d50ff92d63819c9f237bd37357d377fa9c3f189ae41bd1b2a4bc7a8c60dad39",
    "fwd_pp_kernel": {"mfma_busy": 0.669, "traffic": 571300000},
    "bwd_preprocess_kernel": {"mfma_busy": None, "traffic": 293700000},
    "bwd_dkdv_ws_kernel": {"mfma_busy": 0.52, "traffic": 1927700000},
    "bwd_dq_kernel": {"mfma_busy": 0.69, "traffic": 707400000},
}

def kernel_sources_sha():
    import hashlib
    h = hashlib.sha256()
    for name in ("fwd_mfma.hip", "bwd_mfma.hip", "common.hpp", "tile_io.hpp"):
        with open(os.path.join(ROOT, "exact_tiled_attention_07_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_table(w, f_fwd, f_bwd, ms):
    """Per-kernel figures for one step.  Algorithmic FLOP per launch: the
    forward kernel does both forward products; the backward's five products
    per visible pair (S = QK^T again, dP = dO V^T, dV = P^T dO, dK = dS^T Q,
    dQ = dS K) split 4 to the dK/dV kernel and 1 to the dQ kernel (which also
    recomputes S and dP: work that is not counted).  The preprocess kernel is
    rated against HBM: it reads dO and O and the LSE and writes two float32
    rows statistics per query row (padded to 128 rows)."""
    e = 2
    rows = w.batch * w.nheads_q * w.seqlen
    rows_pad = w.batch * w.nheads_q * (-(-w.seqlen // 128) * 128)
    prep_bytes = 2 * rows * w.headdim * e + 4 * rows + 2 * 4 * rows_pad
    spec = [
        ("fwd_pp_kernel<BF16,128,64> (fa_fwd)", "mfma", f_fwd),
        ("bwd_preprocess_kernel<2> (fa_bwd_stage PREPARE)", "hbm", prep_bytes),
        ("bwd_dkdv_ws_kernel<BF16,128,64> (fa_bwd_stage DKDV)", "mfma", 0.8 * f_bwd),
        ("bwd_dq_kernel<BF16,128,64,8> (fa_bwd_stage DQ)", "mfma", 0.2 * f_bwd),
    ]
    out = []
    sha = kernel_sources_sha()
    for (name, bound, work), t in zip(spec, ms):
        if bound == "mfma":
            ach, peak, unit = work / (t * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = work / (t * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
        row = {"kernel": name, "ms": round(t, 4), "bound": bound, "achieved": round(ach, 2), "peak": peak,
               "unit": unit, "frac": round(ach / peak, 4), "mfma_busy": None, "traffic": None}
        c = COUNTERS.get(name.split("<")[0]) if COUNTERS["sources_sha256"] == sha else None
        if c:
            row["mfma_busy"] = c.get("mfma_busy")
            row["traffic"] = c.get("traffic")
        out.append(row)
    return out


def cpu_baseline(w, q, k, v, do, budget_s):
    """Time the float64 oracle on whole heads of the workload until budget_s is
    reached (at least one head, at most one kv group); report TFLOP/s."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=None)
    except Exception:  # pragma: no cover
        blas_threads = None
    G = w.nheads_q // w.nheads_kv
    done, t_total = 0, 0.0
    for b in range(w.batch):
        for h in range(w.nheads_q):
            g = h // G
            kf = k[b:b + 1, :, g:g + 1].double().numpy()
            vf = v[b:b + 1, :, g:g + 1].double().numpy()
            qf = q[b:b + 1, :, h:h + 1].double().numpy()
            dof = do[b:b + 1, :, h:h + 1].double().numpy()
            t0 = time.perf_counter()
            oracle.attention_fwd(qf, kf, vf, causal=w.causal, window=w.window)
            oracle.attention_bwd(dof, qf, kf, vf, causal=w.causal, window=w.window)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    f_head = sum(flops(w)) / (w.batch * w.nheads_q)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": f_head * done / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{done} of {w.batch * w.nheads_q} (batch, query head) pairs x {w.seqlen} rows, fwd+bwd, float64 "
                  f"NumPy oracle ({t_total:.1f} s; {len(os.sched_getaffinity(0))} cores in affinity mask, "
                  f"CPU: {cpu_model})",
    }


def decode_bytes(w, lens):
    """Algorithmic HBM bytes of one fa_fwd_kvcache call: every visible cache
    row and new row read once (K and V), the new rows written into the cache,
    q read, o / lse written, the lengths read."""
    e = 2
    lk = [min(max(int(x), 0) + w.nq, w.capacity) for x in lens]
    kv_read = sum(lk) * w.nheads_kv * w.headdim * e * 2
    appended = sum(min(w.nq, w.capacity - min(max(int(x), 0), w.capacity)) for x in lens)
    kv_write = appended * w.nheads_kv * w.headdim * e * 2
    qo = 2 * w.batch * w.nq * w.nheads_q * w.headdim * e
    return kv_read + kv_write + qo + w.batch * w.nheads_q * w.nq * 4 + w.batch * 4


def decode_leg(calls):
    """Times fa_fwd_kvcache on the benchmark's decode workload."""
    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.workloads import BENCH_DECODE_WORKLOAD, DECODE_WORKLOADS, make_decode_inputs

    w = DECODE_WORKLOADS[BENCH_DECODE_WORKLOAD]
    dev = torch.device("cuda:0")
    q, kc, vc, kn, vn, lens = (t.to(dev) for t in make_decode_inputs(w))
    kw = dict(causal=w.causal, window_size=w.window)
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.nheads_q, w.nq), dtype=torch.float32, device=dev)
    params = fa.make_kv_params(q, kc, vc, out, kn, vn, **kw)
    ws = torch.empty(fa.kvcache_workspace_size(params), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        # The lengths stay fixed, so every call appends the same rows again and
        # attends to the same keys: identical work per call.
        fa.fwd_kvcache(q, kc, vc, lens, kn, vn, out=out, lse=lse, workspace=ws, **kw)

    for _ in range(10):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(calls):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / calls
    nbytes = decode_bytes(w, lens.tolist())
    gbs = nbytes / (us * 1e-6) / 1e9

    # The same call over a paged cache: 256-row pages in a shuffled pool,
    # stored head-major inside each page (num_pages, Hkv, 256, d).
    ps = 256
    per = w.capacity // ps
    n_pages = w.batch * per
    g = torch.Generator("cpu").manual_seed(w.seed)
    table = torch.randperm(n_pages, generator=g).to(torch.int32).reshape(w.batch, per).to(dev)
    kp = torch.empty((n_pages, w.nheads_kv, ps, w.headdim), dtype=q.dtype, device=dev)
    vp = torch.empty_like(kp)
    kpv, vpv = kp.permute(0, 2, 1, 3), vp.permute(0, 2, 1, 3)  # (num_pages, page_size, Hkv, d) views
    for b in range(w.batch):
        for p in range(per):
            kpv[table[b, p]] = kc[b, p * ps:(p + 1) * ps]
            vpv[table[b, p]] = vc[b, p * ps:(p + 1) * ps]

    def call_paged():
        fa.fwd_kvcache_paged(q, kpv, vpv, lens, table, kn, vn, out=out, lse=lse, workspace=ws, **kw)

    for _ in range(10):
        call_paged()
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(calls):
        call_paged()
    ev[1].record(stream)
    torch.cuda.synchronize()
    us_paged = ev[0].elapsed_time(ev[1]) * 1e3 / calls
    return {
        "workload": w.name, "entry_point": "fa_fwd_kvcache",
        "config": {"batch": w.batch, "new_tokens": w.nq, "nheads_q": w.nheads_q, "nheads_kv": w.nheads_kv,
                   "headdim": w.headdim, "capacity": w.capacity, "cache_seqlens": lens.tolist(),
                   "cache_layout": w.kv_layout, "causal": w.causal, "num_splits": "auto"},
        "calls": calls, "us_per_call": round(us, 2),
        "paged": {"page_size": ps, "layout": "shuffled page pool, head-major pages", "us_per_call": round(us_paged, 2),
                  "achieved_GBps": round(nbytes / (us_paged * 1e-6) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes,
                     "timed": "whole call (split + merge kernels), events on the launch stream"},
    }


# Sequence lengths of the packed-batch leg: 16384 tokens, as many as the
# benchmark workload's two sequences of 8192, in a ragged mix.
VARLEN_LENGTHS = [4096, 2560, 2048, 1792, 1536, 1280, 1024, 768, 512, 384, 256, 128]


def next_rows_leg(steps):
    """fwd + bwd throughput of two rows beyond the benchmark step, same heads
    and head size (Hq=32, Hkv=8, d=128, bf16, causal), events on the launch
    stream: a packed batch of VARLEN_LENGTHS through fa_fwd_varlen /
    fa_bwd_varlen, and the benchmark workload with ALiBi slopes and a softcap
    (the modifier kernels).  FLOP per causal sequence of length L: 4*Hq*d*L^2/2
    forward, 2.5 times that backward."""
    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.workloads import BENCH_WORKLOAD, WORKLOADS, make_inputs

    w = WORKLOADS[BENCH_WORKLOAD]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def timed(fwd_call, bwd_call):
        for _ in range(3):
            fwd_call()
            bwd_call()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for e in ev:
            e[0].record(stream)
            fwd_call()
            e[1].record(stream)
            bwd_call()
            e[2].record(stream)
        torch.cuda.synchronize()
        return (sum(e[0].elapsed_time(e[1]) for e in ev) / steps, sum(e[1].elapsed_time(e[2]) for e in ev) / steps)

    def entry(f_fwd, fwd_ms, bwd_ms):
        tf = 3.5 * f_fwd / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
        return {"fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
                "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2), "tflops": round(tf, 2),
                "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}

    out = {"steps": steps}
    # Packed batch.
    g = torch.Generator("cpu").manual_seed(w.seed + 17)
    tot = sum(VARLEN_LENGTHS)
    q, k, v, do = ((torch.randn((tot, h, w.headdim), generator=g) * sd).to(torch.bfloat16).to(dev)
                   for h, sd in ((w.nheads_q, w.sigma), (w.nheads_kv, w.sigma), (w.nheads_kv, w.sigma),
                                 (w.nheads_q, 1.0)))
    cu = torch.tensor([0] + [int(x) for x in torch.tensor(VARLEN_LENGTHS).cumsum(0)], dtype=torch.int32, device=dev)
    mx = max(VARLEN_LENGTHS)
    o = torch.empty_like(q)
    lse = torch.empty((w.nheads_q, tot), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    vp = fa.make_varlen_params(q, k, v, o, mx, mx, causal=True, batch=len(VARLEN_LENGTHS))
    vws = torch.empty(fa.bwd_varlen_workspace_size(vp), dtype=torch.uint8, device=dev)
    fm, bm = timed(lambda: fa.fwd_varlen(q, k, v, cu, cu, mx, mx, causal=True, out=o, lse=lse),
                   lambda: fa.bwd_varlen(do, q, k, v, o, lse, cu, cu, mx, mx, causal=True, dq=dq, dk=dk, dv=dv,
                                         workspace=vws))
    f_fwd = 4.0 * w.nheads_q * w.headdim * sum(L * L / 2 for L in VARLEN_LENGTHS)
    out["varlen"] = {"entry_points": "fa_fwd_varlen + fa_bwd_varlen", "seqlens": VARLEN_LENGTHS,
                     **entry(f_fwd, fm, bm)}
    del q, k, v, do, o, lse, dq, dk, dv, vws
    # Score modifiers on the benchmark workload.
    q, k, v, do = (t.to(dev) for t in make_inputs(w))
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / w.nheads_q) for h in range(w.nheads_q)], dtype=torch.float32,
                          device=dev)
    softcap = 30.0
    kw = dict(causal=True, alibi_slopes=slopes, softcap=softcap)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.nheads_q, w.seqlen), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_workspace_size(fa.make_params(q, k, v, o, **kw)), dtype=torch.uint8, device=dev)
    fm, bm = timed(lambda: fa.fwd(q, k, v, out=o, lse=lse, **kw),
                   lambda: fa.bwd(do, q, k, v, o, lse, dq=dq, dk=dk, dv=dv, workspace=ws, **kw))
    f_fwd = flops(w)[0]
    out["modifiers"] = {"workload": w.name, "alibi_slopes": "2^(-8(h+1)/Hq) per head", "softcap": softcap,
                        **entry(f_fwd, fm, bm)}
    return out


def configs_leg(calls, repeats=5, min_ms=2.0, max_calls=2000):
    """fa_fwd alone and fa_bwd alone (on the forward's outputs) on every named
    workload at its full size, inputs resident in HBM, outputs preallocated,
    no cache flush between calls: warm-up calls, then `repeats` runs of
    max(`calls`, about `min_ms` of work) calls between two events on the
    launch stream; the median run's average per call.  fp16/bf16 rates are
    set against the dense MFMA peak; the fp32 path runs on the vector ALU and
    is not rated."""
    import statistics

    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.workloads import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    out = {"min_calls_per_repeat": calls, "min_ms_per_repeat": min_ms, "repeats": repeats,
           "statistic": "median of repeats", "cache": "not flushed between calls"}
    for name, w in WORKLOADS.items():
        q, k, v, do = (t.to(dev) for t in make_inputs(w))
        kw = dict(causal=w.causal, window_size=w.window)
        o = torch.empty_like(q)
        lse = torch.empty((w.batch, w.nheads_q, w.seqlen), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.bwd_workspace_size(fa.make_params(q, k, v, o, **kw)), dtype=torch.uint8, device=dev)

        def fwd():
            fa.fwd(q, k, v, out=o, lse=lse, **kw)

        def bwd():
            fa.bwd(do, q, k, v, o, lse, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

        def time_it(fn):
            # 3 warm-up calls, then 10 timed ones that size the repeats: each
            # repeat holds at least `calls` calls and at least min_ms of work, so
            # that the latency of the first launch does not dominate small
            # workloads.
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            est = e0.elapsed_time(e1) / 10
            n = max(calls, min(max_calls, math.ceil(min_ms / max(est, 1e-3))))
            runs = []
            for _ in range(repeats):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(n):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                runs.append(e0.elapsed_time(e1) / n)
            return statistics.median(runs), n

        f_fwd, f_bwd = flops(w)
        rated = w.dtype != "fp32"
        entry = {"dtype": w.dtype, "shape": [w.batch, w.seqlen, w.nheads_q, w.nheads_kv, w.headdim],
                 "causal": w.causal, "window": list(w.window), "sigma": w.sigma}
        fm, n = time_it(fwd)
        entry.update(fwd_ms=round(fm, 4), fwd_tflops=round(f_fwd / (fm * 1e-3) / 1e12, 2), fwd_calls=n)
        if rated:
            entry["fwd_frac"] = round(f_fwd / (fm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if w.backward:
            fwd()
            bm, n = time_it(bwd)
            entry.update(bwd_ms=round(bm, 4), bwd_tflops=round(f_bwd / (bm * 1e-3) / 1e12, 2), bwd_calls=n)
            tf = (f_fwd + f_bwd) / ((fm + bm) * 1e-3) / 1e12
            entry["fwd_bwd_tflops"] = round(tf, 2)
            if rated:
                entry["bwd_frac"] = round(f_bwd / (bm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                entry["fwd_bwd_frac"] = round(tf / PEAK_BF16_TFLOPS, 4)
        assert torch.isfinite(o).all()
        out[name] = entry
        del q, k, v, do, o, lse, dq, dk, dv, ws
    return out


def standard_attention_fwd_bwd(q, k, v, do, scale):
    """Attention the standard way, for the memory comparison only: the full
    score matrix S, P = softmax(S), O = P V, then the backward from the stored
    P (dP, dS of the same size).  (batch, heads, seq, d) bf16 tensors; every
    transposed operand of a batched product is made contiguous first."""
    import torch
    s_ = torch.matmul(q, k.transpose(-2, -1).contiguous()) * scale
    n = s_.shape[-1]
    mask = torch.ones(n, n, dtype=torch.bool, device=q.device).triu(1)
    s_.masked_fill_(mask, float("-inf"))
    p = torch.softmax(s_, dim=-1)
    del s_
    o = torch.matmul(p, v)
    dv = torch.matmul(p.transpose(-2, -1).contiguous(), do)
    dp = torch.matmul(do, v.transpose(-2, -1).contiguous())
    dsum = (do * o).sum(-1, keepdim=True)
    ds = p * (dp - dsum)
    del dp
    dq = torch.matmul(ds, k) * scale
    dk = torch.matmul(ds.transpose(-2, -1).contiguous(), q) * scale
    return o, dq, dk, dv


def memory_leg():
    """Peak device memory of one forward + backward beyond the inputs (q, k, v,
    dO), this library against standard attention that keeps the N x N matrices,
    at the pages' memory-benchmark shape: bf16, hidden 2048 = 16 heads x d 128,
    batch 1, causal, N = 2048 and 4096."""
    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.workloads import random_qkv

    out = {"shape": "bf16, batch 1, 16 heads x d 128, causal", "unit": "MiB beyond the inputs"}
    for n in (2048, 4096):
        q, k, v, do = (t.cuda() for t in random_qkv((1, n, 16, 128), (1, n, 16, 128), "bf16", seed=77))
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        o, lse = fa.fwd(q, k, v, causal=True)
        g = fa.bwd(do, q, k, v, o, lse, causal=True)
        torch.cuda.synchronize()
        ours = torch.cuda.max_memory_allocated() - base
        del o, lse, g
        qh, kh, vh, doh = (t.transpose(1, 2).contiguous() for t in (q, k, v, do))
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        r = standard_attention_fwd_bwd(qh, kh, vh, doh, 1.0 / 128 ** 0.5)
        torch.cuda.synchronize()
        std = torch.cuda.max_memory_allocated() - base
        del r, qh, kh, vh, doh
        out[f"N{n}"] = {"this_library": round(ours / 2 ** 20, 1), "standard": round(std / 2 ** 20, 1),
                        "ratio": round(std / ours, 1)}
    return out


def gemm_leg(n=8192, reps=20):
    """Context for the MFMA roofline: the vendor library's bf16 GEMM (torch.matmul,
    which dispatches to hipBLASLt) on n x n x n, timed with events after warm-up.
    It is the dense matrix-core rate the chip sustains under load (clock and power
    included), next to the nameplate peak the roofline uses."""
    import torch

    g = torch.Generator(device="cuda").manual_seed(3)
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda", generator=g)
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda", generator=g)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = 2.0 * n ** 3 / ms / 1e9
    return {"what": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt)", "ms": round(ms, 4), "tflops": round(tflops, 1),
            "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.workloads import BENCH_WORKLOAD, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    w = WORKLOADS[BENCH_WORKLOAD]
    q_c, k_c, v_c, do_c = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (q_c, k_c, v_c, do_c))
    kw = dict(causal=w.causal, window_size=w.window)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.nheads_q, w.seqlen), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    params = fa.make_params(q, k, v, o, **kw)
    ws = torch.empty(fa.bwd_workspace_size(params), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    stages = (fa.FA_BWD_PREPARE, fa.FA_BWD_DKDV, fa.FA_BWD_DQ)

    def step(ev=None):
        # fa_fwd, then fa_bwd as its three stages (bitwise the same as one
        # fa_bwd call), with an event between launches so that every kernel is
        # timed on the stream it runs on.
        if ev is not None:
            ev[0].record(stream)
        fa.fwd(q, k, v, out=o, lse=lse, **kw)
        for i, st in enumerate(stages):
            if ev is not None:
                ev[1 + i].record(stream)
            fa.bwd(do, q, k, v, o, lse, dq=dq, dk=dk, dv=dv, workspace=ws, stage=st, **kw)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert torch.isfinite(o).all() and torch.isfinite(dq).all()

    def avg_ms(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in events) / len(events)

    f_fwd, f_bwd = flops(w)
    ms_per_step = wall * 1e3 / args.steps
    value = (f_fwd + f_bwd) * args.steps / wall / 1e12
    fwd_avg, bwd_avg, step_avg = avg_ms(0, 1), avg_ms(1, 4), avg_ms(0, 4)
    kernels = kernel_table(w, f_fwd, f_bwd, [avg_ms(i, i + 1) for i in range(4)])
    dom = max(kernels, key=lambda r: r["ms"])
    roof = {
        "kernel": dom["kernel"],
        "bound": dom["bound"],
        "achieved": dom["achieved"],
        "peak": dom["peak"],
        "unit": dom["unit"],
        "frac": dom["frac"],
        "mfma_busy": dom.get("mfma_busy"),
        "traffic": dom.get("traffic"),
    }

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v, dO; shapes of the pages' workloads)",
        "config": {
            "workload": w.name, "passes": "fwd+bwd", "batch": w.batch, "seqlen": w.seqlen,
            "nheads_q": w.nheads_q, "nheads_kv": w.nheads_kv, "headdim": w.headdim,
            "causal": w.causal, "window": list(w.window), "parallelism": "single GPU",
        },
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(fwd_avg, 4),
        "bwd_ms": round(bwd_avg, 4),
        "fwd_tflops": round(f_fwd / (fwd_avg * 1e-3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / (bwd_avg * 1e-3) / 1e12, 2),
        "event_ms_per_step": round(step_avg, 4),
        "roofline": roof,
        "kernels": kernels,
    }
    if args.decode_calls > 0:
        out["decode"] = decode_leg(args.decode_calls)
    if args.next_rows_steps > 0:
        out["next_rows"] = next_rows_leg(args.next_rows_steps)
    if args.config_calls > 0:
        out["configs"] = configs_leg(args.config_calls)
    if not args.no_memory:
        out["memory"] = memory_leg()
    if not args.no_gemm:
        out["gemm_reference"] = gemm_leg()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q_c, k_c, v_c, do_c, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
