"""Exact tiled attention for AMD MI355X (gfx950).

O = softmax(scale * Q K^T + causal/window mask) V, computed tile by tile with an
online softmax in hand-written HIP kernels (32x32x16 MFMA for fp16/bf16, vector
ALU for fp32), behind the C ABI of include/fa.h.  This package is the thin
Python binding: torch provides device memory and streams only.

    o, lse = fwd(q, k, v, causal=True)
    dq, dk, dv = bwd(do, q, k, v, o, lse, causal=True)
    o = attention(q, k, v, causal=True)          # autograd wrapper
    o, lse = fwd_kvcache(q, k_cache, v_cache, cache_seqlens, k_new, v_new, causal=True)
    o, lse = fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_q, max_k)   # packed batch
    o = attention_qkvpacked(qkv, causal=True)    # qkv (batch, seqlen, 3, nheads, headdim)
"""

from ._native import (  # noqa: F401
    FA_BF16, FA_BWD_DKDV, FA_BWD_DQ, FA_BWD_PREPARE, FA_ERR_HIP, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED,
    FA_F16, FA_F32, FA_OK, SIGNATURES,
    FaError, FaKvParams, FaParams, FaVarlenParams, attention, attention_qkvpacked, attention_varlen, bwd, bwd_noalloc,
    bwd_varlen, bwd_varlen_workspace_size, bwd_workspace_size, fwd, fwd_kvcache, fwd_kvcache_paged, fwd_qkvpacked,
    fwd_varlen,
    kvcache_workspace_size, library_path, load_library, make_kv_params, make_params, make_varlen_params, version,
)
