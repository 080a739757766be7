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


def random_qkv(shape_q, shape_kv, dtype, seed, sigma=1.0):
    """Same recipe for an arbitrary shape (test sweeps)."""
    g = torch.Generator("cpu").manual_seed(seed)
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    q = (torch.randn(shape_q, generator=g, dtype=torch.float32) * sigma).to(dt)
    k = (torch.randn(shape_kv, generator=g, dtype=torch.float32) * sigma).to(dt)
    v = (torch.randn(shape_kv, generator=g, dtype=torch.float32) * sigma).to(dt)
    do = torch.randn(shape_q, generator=g, dtype=torch.float32).to(dt)
    return q, k, v, do
