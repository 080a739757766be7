"""Seeded synthetic inputs for the attention workloads.

This module only draws random tensors and names shapes; it holds none of the
attention arithmetic, so both the oracle-side checks and the GPU path can take
their inputs from it.

The shapes follow the workloads the pages benchmark: random Q/K/V in the layout
(batch, seqlen, nheads, headdim) ([P4] "FlashAttention 实战指南", section "上手
FlashAttention 的三步走"), fp16/bf16 with head dimension 64 or 128, hidden size
2048 and sequence lengths from 512 to 16k ([P4] section "实测数据"), and the
(2, 32, 8192, 128) timing shape of [P5] "AI模型推理优化Flash Attention原理",
section "进阶一点的用法".

Decode workloads follow [P4] section "增量解码场景flash_attn_with_kvcache": a
few new queries per batch entry against a long KV cache whose valid length
(cache_seqlens) differs between entries, at low batch and long context.
"""

from dataclasses import dataclass, field

import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    batch: int
    seqlen: int
    nheads_q: int
    nheads_kv: int
    headdim: int
    causal: bool
    window: tuple = (-1, -1)
    sigma: float = 1.0          # std of q, k, v (dO always has std 1)
    backward: bool = True
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def q_shape(self):
        return (self.batch, self.seqlen, self.nheads_q, self.headdim)

    @property
    def kv_shape(self):
        return (self.batch, self.seqlen, self.nheads_kv, self.headdim)


WORKLOADS = {
    "fp32_b1_h2_n128_d64": Workload(
        "fp32_b1_h2_n128_d64", "fp32", 1, 128, 2, 2, 64, False, backward=False, seed=1001),
    "fp16_b2_h16_n512_d64_causal": Workload(
        "fp16_b2_h16_n512_d64_causal", "fp16", 2, 512, 16, 16, 64, True, seed=1002),
    "bf16_b2_h16_n4096_d128_causal": Workload(
        "bf16_b2_h16_n4096_d128_causal", "bf16", 2, 4096, 16, 16, 128, True, seed=1003),
    "bf16_b2_hq32_hkv8_n8192_d128_causal": Workload(
        "bf16_b2_hq32_hkv8_n8192_d128_causal", "bf16", 2, 8192, 32, 8, 128, True, seed=1004),
    "bf16_b2_hq32_hkv8_n8192_d128_window1024": Workload(
        "bf16_b2_hq32_hkv8_n8192_d128_window1024", "bf16", 2, 8192, 32, 8, 128, True,
        window=(1024, 0), backward=False, seed=1004),
    "bf16_b1_h16_n16384_d128_causal_sigma05": Workload(
        "bf16_b1_h16_n16384_d128_causal_sigma05", "bf16", 1, 16384, 16, 16, 128, True,
        sigma=0.5, seed=1005),
}

# The workload the benchmark times (fwd + bwd on it).
BENCH_WORKLOAD = "bf16_b2_hq32_hkv8_n8192_d128_causal"


def make_inputs(w: Workload, seed=None, batch=None, seqlen=None):
    """Draw q, k, v, dO on the CPU: float32 N(0, sigma^2) (dO: N(0, 1)), drawn
    in that order from one seeded generator, then rounded to the workload dtype.
    ``batch`` / ``seqlen`` override the shape (same recipe, smaller case)."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    b = w.batch if batch is None else batch
    n = w.seqlen if seqlen is None else seqlen
    qs = (b, n, w.nheads_q, w.headdim)
    ks = (b, n, w.nheads_kv, w.headdim)
    dt = DTYPES[w.dtype]
    q = (torch.randn(qs, generator=g, dtype=torch.float32) * w.sigma).to(dt)
    k = (torch.randn(ks, generator=g, dtype=torch.float32) * w.sigma).to(dt)
    v = (torch.randn(ks, generator=g, dtype=torch.float32) * w.sigma).to(dt)
    do = torch.randn(qs, generator=g, dtype=torch.float32).to(dt)
    return q, k, v, do


def random_qkv(shape_q, shape_kv, dtype, seed, sigma=1.0, sigma_v=None):
    """Same recipe for an arbitrary shape (test sweeps); ``sigma_v`` (default
    ``sigma``) sets the std of v alone."""
    g = torch.Generator("cpu").manual_seed(seed)
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    sv = sigma if sigma_v is None else sigma_v
    q = (torch.randn(shape_q, generator=g, dtype=torch.float32) * sigma).to(dt)
    k = (torch.randn(shape_kv, generator=g, dtype=torch.float32) * sigma).to(dt)
    v = (torch.randn(shape_kv, generator=g, dtype=torch.float32) * sv).to(dt)
    do = torch.randn(shape_q, generator=g, dtype=torch.float32).to(dt)
    return q, k, v, do


def monotone_key_qkv(shape_q, shape_kv, dtype, seed, rise_per_key, q_gain=1.0):
    """Inputs whose scaled scores climb along the keys: k_j = (j / N) * c * u +
    0.1 * noise and q_i = q_gain * u + 0.5 * noise, with u a random N(0, 1)
    direction, so that q_i . u is about q_gain * headdim > 0 for every query.
    The scaled score q_i . k_j / sqrt(headdim) then grows by about
    ``rise_per_key`` (natural-log units) from one key to the next
    (c = rise_per_key * N / (q_gain * sqrt(headdim))), so a running row maximum
    taken tile by tile rises on every tile; q_gain moves magnitude from the
    keys to the queries.  v and dO are N(0, 1).  All drawn from one seeded CPU
    generator, then rounded to dtype."""
    g = torch.Generator("cpu").manual_seed(seed)
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    b, n, hq, d = shape_q
    _, nk, hkv, _ = shape_kv
    u = torch.randn((d,), generator=g, dtype=torch.float32)
    c = rise_per_key * nk / (q_gain * d ** 0.5)
    ramp = (torch.arange(nk, dtype=torch.float32) / nk)[None, :, None, None]
    k = ramp * c * u + 0.1 * torch.randn(shape_kv, generator=g, dtype=torch.float32)
    q = q_gain * u + 0.5 * torch.randn(shape_q, generator=g, dtype=torch.float32)
    v = torch.randn(shape_kv, generator=g, dtype=torch.float32)
    do = torch.randn(shape_q, generator=g, dtype=torch.float32)
    return q.to(dt), k.to(dt), v.to(dt), do.to(dt)


@dataclass(frozen=True)
class DecodeWorkload:
    """Queries against a KV cache: Nq new rows per batch entry, appended first.

    The valid cache lengths before the append are drawn uniformly from
    [min_len, max_len] (a ragged length mix); cache rows past them hold random
    values that the result must not depend on."""
    name: str
    dtype: str
    batch: int
    nq: int
    nheads_q: int
    nheads_kv: int
    headdim: int
    capacity: int
    min_len: int
    max_len: int
    causal: bool = True
    window: tuple = (-1, -1)
    seed: int = 0
    # Cache storage order: "bshd" stores (batch, capacity, heads, headdim);
    # "bhsd" stores (batch, heads, capacity, headdim), so the 32 rows of a key
    # tile of one head are one contiguous 8 KB block (d = 128).  Both are
    # handed over as (batch, capacity, heads, headdim) views with strides.
    kv_layout: str = "bshd"
    notes: str = field(default="", compare=False)


DECODE_WORKLOADS = {
    "bf16_decode_b8_hq32_hkv8_d128_cap16384": DecodeWorkload(
        "bf16_decode_b8_hq32_hkv8_d128_cap16384", "bf16", 8, 1, 32, 8, 128, 16384, 8192, 16383, seed=2001,
        kv_layout="bhsd", notes="one new token per entry, GQA 4, long ragged context, head-major cache"),
    "fp16_decode_b4_hq16_hkv16_d64_cap4096_nq4": DecodeWorkload(
        "fp16_decode_b4_hq16_hkv16_d64_cap4096_nq4", "fp16", 4, 4, 16, 16, 64, 4096, 1, 4092, seed=2002,
        notes="four new tokens per entry (multi-token decode), MHA"),
    "bf16_chunk_b2_hq32_hkv8_d128_cap8192_nq64": DecodeWorkload(
        "bf16_chunk_b2_hq32_hkv8_d128_cap8192_nq64", "bf16", 2, 64, 32, 8, 128, 8192, 0, 8128, seed=2003,
        notes="chunked prefill: 64 new tokens against the cache"),
}

# The decode workload the benchmark times beside the training step.
BENCH_DECODE_WORKLOAD = "bf16_decode_b8_hq32_hkv8_d128_cap16384"


def make_decode_inputs(w: DecodeWorkload, seed=None, batch=None, capacity=None):
    """Draw q, k_cache, v_cache, k_new, v_new (float32 N(0, 1) rounded to the
    workload dtype) and cache_seqlens (int32, uniform in [min_len, max_len]
    clipped to capacity - nq) from one seeded CPU generator, in that order.
    ``batch`` / ``capacity`` override the shape (same recipe, smaller case; the
    length bounds scale with the capacity)."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    b = w.batch if batch is None else batch
    cap = w.capacity if capacity is None else capacity
    dt = DTYPES[w.dtype]
    q = torch.randn((b, w.nq, w.nheads_q, w.headdim), generator=g, dtype=torch.float32).to(dt)
    kc = torch.randn((b, cap, w.nheads_kv, w.headdim), generator=g, dtype=torch.float32).to(dt)
    vc = torch.randn((b, cap, w.nheads_kv, w.headdim), generator=g, dtype=torch.float32).to(dt)
    if w.kv_layout == "bhsd":
        kc = kc.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        vc = vc.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    elif w.kv_layout != "bshd":
        raise ValueError(f"unknown cache layout {w.kv_layout}")
    kn = torch.randn((b, w.nq, w.nheads_kv, w.headdim), generator=g, dtype=torch.float32).to(dt)
    vn = torch.randn((b, w.nq, w.nheads_kv, w.headdim), generator=g, dtype=torch.float32).to(dt)
    lo_w, hi_w = w.min_len * cap // w.capacity, w.max_len * cap // w.capacity
    hi = max(0, min(hi_w, cap - w.nq))
    lo = min(lo_w, hi)
    lens = torch.randint(lo, hi + 1, (b,), generator=g, dtype=torch.int64).to(torch.int32)
    return q, kc, vc, kn, vn, lens
