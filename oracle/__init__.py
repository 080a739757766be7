"""CPU float64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library or its Python
binding, and it imports neither.

Sources (the web pages this method is taken from, cited by title and section):

* [P4] "FlashAttention 实战指南:如何把训练内存省 20 倍、速度提 4 倍" (kwkr.cn) --
  section "长序列注意力为什么会爆内存" (standard attention in three steps:
  Q times K transposed, a row softmax, then times V), section "上手 FlashAttention
  的三步走" (tensor layout (batch, seqlen, nheads, headdim) and the causal flag),
  section "进阶参数如何配置causal、window_size 与 MQA/GQA" (window_size
  (left, right) with -1 meaning unbounded; fewer K/V heads than Q heads, the Q head
  count an integer multiple of the K/V head count).
* [P4] same page, section "增量解码场景flash_attn_with_kvcache" (new keys and
  values appended to a cache in place, cache_seqlens as each batch entry's valid
  length) -- ``kvcache.py``.
* [P4] same page, section "上手 FlashAttention 的三步走" (the varlen interfaces
  for batches of sequences of different lengths) -- ``varlen.py``.
* [P5] "AI模型推理优化Flash Attention原理" (52runoob.com) -- section "先搞清楚原理"
  (the standard_attention listing: scores scaled by one over the square root of
  the head dimension, softmax over the key axis, product with V).

Every function here is the plain definition written out in float64: the full
score row is materialised, soft-maxed and multiplied by V.  There is no tiling,
no online softmax and no fusion.  Parity of every function is pinned by
``tests/test_oracle.py`` (brute force, closed forms, invariants, finite
differences, a hand-derived golden example and a float64 library cross-check);
no function here is "parity unpinned".
"""

from .attention import ALL_FUNCTIONS as _ATTENTION_FUNCTIONS
from .attention import (  # noqa: F401
    attention_bwd,
    attention_fwd,
    attention_fwd_rows,
    head_of,
    masked_softmax,
    modified_logits,
    scores,
    slope_of,
    visible,
)
from .kvcache import ALL_FUNCTIONS as _KVCACHE_FUNCTIONS
from .kvcache import kvcache_fwd, kvcache_fwd_paged  # noqa: F401
from .varlen import ALL_FUNCTIONS as _VARLEN_FUNCTIONS
from .varlen import attention_bwd_varlen, attention_fwd_varlen  # noqa: F401

ALL_FUNCTIONS = _ATTENTION_FUNCTIONS + _KVCACHE_FUNCTIONS + _VARLEN_FUNCTIONS
