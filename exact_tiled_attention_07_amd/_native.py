"""ctypes binding of libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the attention computation runs in the library's HIP
kernels.  There is no CPU path: tensors must live on a GPU, and a missing
library raises instead of falling back.
"""

import ctypes
import math
import os

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_BWD_PREPARE, FA_BWD_DKDV, FA_BWD_DQ = 0, 1, 2
_TORCH_DTYPE = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}

# Every function the header declares, with its ctypes signature.
_I64x3 = ctypes.c_int64 * 3


class FaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen_q", ctypes.c_int64),
        ("seqlen_k", ctypes.c_int64),
        ("nheads_q", ctypes.c_int64),
        ("nheads_kv", ctypes.c_int64),
        ("headdim", ctypes.c_int64),
        ("q_strides", _I64x3),
        ("k_strides", _I64x3),
        ("v_strides", _I64x3),
        ("o_strides", _I64x3),
        ("dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("alibi_slopes", ctypes.c_void_p),
        ("alibi_batch_stride", ctypes.c_int64),
        ("softcap", ctypes.c_float),
        ("reserved_mod", ctypes.c_int32),
    ]


class FaVarlenParams(ctypes.Structure):
    _fields_ = [
        ("base", FaParams),
        ("total_q", ctypes.c_int64),
        ("total_k", ctypes.c_int64),
    ]


class FaKvParams(ctypes.Structure):
    _fields_ = [
        ("base", FaParams),
        ("knew_strides", _I64x3),
        ("vnew_strides", _I64x3),
        ("num_splits", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_P = ctypes.POINTER(FaParams)
_PK = ctypes.POINTER(FaKvParams)
_PV = ctypes.POINTER(FaVarlenParams)
_V = ctypes.c_void_p
SIGNATURES = {
    "fa_fwd": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V]),
    "fa_bwd_workspace_size": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "fa_bwd": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "fa_bwd_stage": (ctypes.c_int, [_P, ctypes.c_int, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t,
                                    _V]),
    "fa_bwd_noalloc": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V]),
    "fa_fwd_varlen": (ctypes.c_int, [_PV, _V, _V, _V, _V, _V, _V, _V, _V]),
    "fa_bwd_varlen_workspace_size": (ctypes.c_int, [_PV, ctypes.POINTER(ctypes.c_size_t)]),
    "fa_bwd_varlen": (ctypes.c_int, [_PV, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "fa_fwd_kvcache_workspace_size": (ctypes.c_int, [_PK, ctypes.POINTER(ctypes.c_size_t)]),
    "fa_fwd_kvcache": (ctypes.c_int, [_PK, _V, _V, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "fa_fwd_kvcache_paged": (ctypes.c_int, [_PK, ctypes.c_int32, ctypes.c_int64, _V, ctypes.c_int64, _V, _V, _V, _V,
                                            _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "fa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_version": (ctypes.c_int, []),
}

_lib = None


class FaError(RuntimeError):
    """A non-OK fa_status returned by the library."""

    def __init__(self, status, detail):
        self.status = status
        self.detail = detail
        super().__init__(f"{_status_name(status)}: {detail}")


def _status_name(status):
    return {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED", 3: "FA_ERR_HIP"}.get(
        status, f"status {status}")


def library_path():
    return LIB_PATH


def load_library():
    """Load libfa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m exact_tiled_attention_07_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def version():
    return load_library().fa_version()


def _check(status):
    if status != FA_OK:
        lib = load_library()
        raise FaError(status, lib.fa_last_error().decode(errors="replace"))


def _strides3(t):
    s = t.stride()
    return _I64x3(s[0], s[1], s[2])


def _set_modifiers(p, nheads_q, batch, alibi_slopes, softcap):
    """Score modifiers: alibi_slopes a float32 GPU tensor (nheads_q,) or
    (batch, nheads_q) (kept alive by the caller for the call), softcap >= 0."""
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or not alibi_slopes.is_cuda or not alibi_slopes.is_contiguous():
            raise ValueError("alibi_slopes must be a contiguous float32 GPU tensor")
        if tuple(alibi_slopes.shape) == (nheads_q,):
            p.alibi_batch_stride = 0
        elif tuple(alibi_slopes.shape) == (batch, nheads_q):
            p.alibi_batch_stride = nheads_q
        else:
            raise ValueError(f"alibi_slopes must be ({nheads_q},) or ({batch}, {nheads_q})")
        p.alibi_slopes = alibi_slopes.data_ptr()
    p.softcap = float(softcap)


def make_params(q, k, v, o, *, causal=False, window_size=(-1, -1), scale=None, alibi_slopes=None, softcap=0.0):
    """FaParams for tensors shaped (batch, seqlen, nheads, headdim)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (batch, seqlen, nheads, headdim)")
    if q.dtype not in _TORCH_DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for t in (k, v, o):
        if t.dtype != q.dtype:
            raise ValueError("q, k, v (and o) must share one dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    b, nq, hq, d = q.shape
    if k.shape[0] != b or k.shape[3] != d or o.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v and o")
    for t in (q, k, v, o):
        if t.stride(3) != 1 and t.shape[3] > 1:
            raise ValueError("the headdim axis must be contiguous (stride 1)")
    wl, wr = window_size
    p = FaParams()
    p.batch, p.seqlen_q, p.seqlen_k = b, nq, k.shape[1]
    p.nheads_q, p.nheads_kv, p.headdim = hq, k.shape[2], d
    p.q_strides, p.k_strides = _strides3(q), _strides3(k)
    p.v_strides, p.o_strides = _strides3(v), _strides3(o)
    p.dtype = _TORCH_DTYPE[q.dtype]
    p.scale = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    p.causal = 1 if causal else 0
    p.window_left, p.window_right = int(wl), int(wr)
    _set_modifiers(p, hq, b, alibi_slopes, softcap)
    return p


# make_params results of recent dense calls, keyed on everything make_params
# reads, with the backward workspace size once it has been asked for.  A call
# with ALiBi slopes carries a device pointer in its parameters and is not kept.
_PARAMS_CACHE = {}
_PARAMS_CACHE_MAX = 256


def _dense_params(q, k, v, o, causal, window_size, scale, alibi_slopes, softcap):
    """[FaParams, workspace bytes or None] for fwd/bwd; the FaParams is shared
    between calls and must not be modified."""
    if alibi_slopes is not None:
        return [make_params(q, k, v, o, causal=causal, window_size=window_size, scale=scale,
                            alibi_slopes=alibi_slopes, softcap=softcap), None]
    key = (q.shape, q.stride(), k.shape, k.stride(), v.shape, v.stride(), o.shape, o.stride(), q.dtype, k.dtype,
           v.dtype, o.dtype, bool(causal), tuple(window_size), None if scale is None else float(scale),
           float(softcap))
    entry = _PARAMS_CACHE.get(key)
    if entry is None:
        entry = [make_params(q, k, v, o, causal=causal, window_size=window_size, scale=scale, softcap=softcap),
                 None]
        if len(_PARAMS_CACHE) >= _PARAMS_CACHE_MAX:
            _PARAMS_CACHE.clear()
        _PARAMS_CACHE[key] = entry
    return entry


def _require_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU (there is no CPU path)")


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(None)


def fwd(q, k, v, *, causal=False, window_size=(-1, -1), scale=None, out=None, lse=None, alibi_slopes=None,
        softcap=0.0):
    """Exact attention forward: returns (o, lse).

    q (B, Nq, Hq, d); k, v (B, Nk, Hkv, d); o like q; lse float32 (B, Hq, Nq).
    alibi_slopes (float32 GPU tensor (Hq,) or (B, Hq)) and softcap are the
    optional score modifiers of include/fa.h.
    """
    _require_gpu(q, k, v)
    lib = load_library()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    p = _dense_params(q, k, v, out, causal, window_size, scale, alibi_slopes, softcap)[0]
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def bwd_workspace_size(params):
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.fa_bwd_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def bwd(dout, q, k, v, out, lse, *, causal=False, window_size=(-1, -1), scale=None,
        dq=None, dk=None, dv=None, workspace=None, stage=None, alibi_slopes=None, softcap=0.0):
    """Exact attention backward: returns (dq, dk, dv) of L = sum(out * dout).

    dout uses out's layout; dq gets q's strides, dk/dv get k's and v's.
    With ``stage`` (FA_BWD_PREPARE, FA_BWD_DKDV or FA_BWD_DQ) only that stage
    of the backward pass runs (fa_bwd_stage); the caller then passes the same
    ``workspace`` to all three stages.
    """
    if stage is not None and workspace is None:
        raise ValueError("a single backward stage needs the caller's workspace")
    _require_gpu(dout, q, k, v, out, lse)
    lib = load_library()
    if dout.shape != q.shape or dout.dtype != q.dtype or dout.stride() != out.stride():
        raise ValueError("dout must have the shape, dtype and strides of out")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[0], q.shape[2], q.shape[1]) \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (batch, nheads_q, seqlen_q) tensor")
    entry = _dense_params(q, k, v, out, causal, window_size, scale, alibi_slopes, softcap)
    p = entry[0]
    dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device) if dv is None else dv
    for g, ref in ((dq, q), (dk, k), (dv, v)):
        if g.shape != ref.shape or g.stride() != ref.stride() or g.dtype != ref.dtype:
            raise ValueError("gradient buffers must match the shape, strides and dtype of q/k/v")
    if entry[1] is None:
        entry[1] = bwd_workspace_size(p)
    need = entry[1]
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ptrs = (_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(workspace), workspace.numel(), _stream(q.device))
    with torch.cuda.device(q.device):
        if stage is None:
            _check(lib.fa_bwd(ctypes.byref(p), *ptrs))
        else:
            _check(lib.fa_bwd_stage(ctypes.byref(p), int(stage), *ptrs))
    return dq, dk, dv


def bwd_noalloc(dout, q, k, v, out, lse, *, causal=False, window_size=(-1, -1), scale=None, dq=None, dk=None,
                dv=None, alibi_slopes=None, softcap=0.0):
    """fa_bwd_noalloc: the backward of :func:`bwd` with the row statistics in
    the library's static per-GPU scratch instead of a workspace.  The library
    allocates nothing; gradient buffers not passed in are allocated here by
    torch, as in :func:`bwd`."""
    _require_gpu(dout, q, k, v, out, lse)
    lib = load_library()
    if dout.shape != q.shape or dout.dtype != q.dtype or dout.stride() != out.stride():
        raise ValueError("dout must have the shape, dtype and strides of out")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[0], q.shape[2], q.shape[1]) \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (batch, nheads_q, seqlen_q) tensor")
    p = make_params(q, k, v, out, causal=causal, window_size=window_size, scale=scale, alibi_slopes=alibi_slopes,
                    softcap=softcap)
    dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device) if dv is None else dv
    for g, ref in ((dq, q), (dk, k), (dv, v)):
        if g.shape != ref.shape or g.stride() != ref.stride() or g.dtype != ref.dtype:
            raise ValueError("gradient buffers must match the shape, strides and dtype of q/k/v")
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_noalloc(ctypes.byref(p), _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _stream(q.device)))
    return dq, dk, dv


def make_varlen_params(q, k, v, o, max_seqlen_q, max_seqlen_k, *, causal=False, window_size=(-1, -1),
                       scale=None, alibi_slopes=None, softcap=0.0, batch=0):
    """FaVarlenParams for packed tensors q/o (total_q, Hq, d), k/v (total_k, Hkv, d)."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or o.dim() != 3:
        raise ValueError("packed q, k, v, o must be 3-D (total, nheads, headdim)")
    if q.dtype not in _TORCH_DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for t in (k, v, o):
        if t.dtype != q.dtype:
            raise ValueError("q, k, v (and o) must share one dtype")
    if k.shape != v.shape or o.shape != q.shape or k.shape[2] != q.shape[2]:
        raise ValueError("shape mismatch between q, k, v and o")
    for t in (q, k, v, o):
        if t.stride(2) != 1 and t.shape[2] > 1:
            raise ValueError("the headdim axis must be contiguous (stride 1)")
    wl, wr = window_size
    p = FaVarlenParams()
    b = p.base
    b.batch = 0  # set by the caller (number of sequences)
    b.seqlen_q, b.seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    b.nheads_q, b.nheads_kv, b.headdim = q.shape[1], k.shape[1], q.shape[2]
    b.q_strides = _I64x3(0, q.stride(0), q.stride(1))
    b.k_strides = _I64x3(0, k.stride(0), k.stride(1))
    b.v_strides = _I64x3(0, v.stride(0), v.stride(1))
    b.o_strides = _I64x3(0, o.stride(0), o.stride(1))
    b.dtype = _TORCH_DTYPE[q.dtype]
    b.scale = (1.0 / math.sqrt(q.shape[2])) if scale is None else float(scale)
    b.causal = 1 if causal else 0
    b.window_left, b.window_right = int(wl), int(wr)
    p.total_q, p.total_k = q.shape[0], k.shape[0]
    b.batch = int(batch)
    _set_modifiers(b, q.shape[1], int(batch), alibi_slopes, softcap)
    return p


def _check_offsets(cu, name):
    if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous() or cu.numel() < 1:
        raise ValueError(f"{name} must be a contiguous 1-D int32 tensor of batch + 1 offsets")


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
               window_size=(-1, -1), scale=None, out=None, lse=None, alibi_slopes=None, softcap=0.0):
    """Forward over a packed batch: returns (o, lse).

    q (total_q, Hq, d); k, v (total_k, Hkv, d); cu_seqlens_* int32 (batch + 1,)
    on the device; max_seqlen_* bound the sequence lengths.  o like q; lse
    float32 (Hq, total_q).
    """
    _require_gpu(q, k, v, cu_seqlens_q, cu_seqlens_k)
    _check_offsets(cu_seqlens_q, "cu_seqlens_q")
    _check_offsets(cu_seqlens_k, "cu_seqlens_k")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    lib = load_library()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    p = make_varlen_params(q, k, v, out, max_seqlen_q, max_seqlen_k, causal=causal, window_size=window_size,
                           scale=scale, alibi_slopes=alibi_slopes, softcap=softcap, batch=cu_seqlens_q.numel() - 1)
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd_varlen(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                 _ptr(cu_seqlens_k), _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def bwd_varlen_workspace_size(params):
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.fa_bwd_varlen_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def bwd_varlen(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *,
               causal=False, window_size=(-1, -1), scale=None, dq=None, dk=None, dv=None, workspace=None,
               alibi_slopes=None, softcap=0.0):
    """Backward over a packed batch: returns (dq, dk, dv) of L = sum(out * dout)."""
    _require_gpu(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k)
    _check_offsets(cu_seqlens_q, "cu_seqlens_q")
    _check_offsets(cu_seqlens_k, "cu_seqlens_k")
    lib = load_library()
    if dout.shape != q.shape or dout.dtype != q.dtype or dout.stride() != out.stride():
        raise ValueError("dout must have the shape, dtype and strides of out")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0]) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (nheads_q, total_q) tensor")
    p = make_varlen_params(q, k, v, out, max_seqlen_q, max_seqlen_k, causal=causal, window_size=window_size,
                           scale=scale, alibi_slopes=alibi_slopes, softcap=softcap, batch=cu_seqlens_q.numel() - 1)
    dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device) if dv is None else dv
    for g, ref in ((dq, q), (dk, k), (dv, v)):
        if g.shape != ref.shape or g.stride() != ref.stride() or g.dtype != ref.dtype:
            raise ValueError("gradient buffers must match the shape, strides and dtype of q/k/v")
    need = bwd_varlen_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_varlen(ctypes.byref(p), _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(workspace), workspace.numel(), _stream(q.device)))
    return dq, dk, dv


def make_kv_params(q, k_cache, v_cache, out, k_new=None, v_new=None, *, causal=False, window_size=(-1, -1),
                   scale=None, num_splits=0, alibi_slopes=None, softcap=0.0):
    """FaKvParams: q/out (B, Nq, Hq, d), caches (B, capacity, Hkv, d), new rows like q with Hkv heads."""
    base = make_params(q, k_cache, v_cache, out, causal=causal, window_size=window_size, scale=scale,
                       alibi_slopes=alibi_slopes, softcap=softcap)
    p = FaKvParams()
    p.base = base
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    if k_new is not None:
        want = (q.shape[0], q.shape[1], k_cache.shape[2], q.shape[3])
        for t in (k_new, v_new):
            if tuple(t.shape) != want or t.dtype != q.dtype:
                raise ValueError(f"k_new / v_new must be {want} of dtype {q.dtype}")
            if t.stride(3) != 1 and t.shape[3] > 1:
                raise ValueError("the headdim axis must be contiguous (stride 1)")
        p.knew_strides, p.vnew_strides = _strides3(k_new), _strides3(v_new)
    p.num_splits = int(num_splits)
    p.reserved = 0
    return p


def kvcache_workspace_size(params):
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.fa_fwd_kvcache_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def fwd_kvcache(q, k_cache, v_cache, cache_seqlens, k_new=None, v_new=None, *, causal=False,
                window_size=(-1, -1), scale=None, num_splits=0, out=None, lse=None, workspace=None,
                alibi_slopes=None, softcap=0.0):
    """Attention of q against a KV cache, appending k_new / v_new first: returns (o, lse).

    q (B, Nq, Hq, d); k_cache, v_cache (B, capacity, Hkv, d), updated in place
    when k_new / v_new (B, Nq, Hkv, d) are given; cache_seqlens int32 (B,) on the
    device, the valid rows before the append.  Query i is aligned to key
    i + Lk - Nq where Lk is the key count after the append.  num_splits = 0
    lets the library choose how many parts the key range is split into.
    """
    _require_gpu(q, k_cache, v_cache, cache_seqlens)
    if k_new is not None:
        _require_gpu(k_new, v_new)
    lib = load_library()
    if cache_seqlens.dtype != torch.int32 or tuple(cache_seqlens.shape) != (q.shape[0],) \
            or not cache_seqlens.is_contiguous():
        raise ValueError("cache_seqlens must be a contiguous int32 tensor of shape (batch,)")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    p = make_kv_params(q, k_cache, v_cache, out, k_new, v_new, causal=causal, window_size=window_size,
                       scale=scale, num_splits=num_splits, alibi_slopes=alibi_slopes, softcap=softcap)
    need = kvcache_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd_kvcache(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
                                  _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse), _ptr(workspace),
                                  workspace.numel(), _stream(q.device)))
    return out, lse


class _Layout:
    """Shape, strides and dtype of a tensor view that is described, not built."""

    def __init__(self, shape, strides, dtype):
        self.shape, self._strides, self.dtype = torch.Size(shape), tuple(strides), dtype

    def dim(self):
        return len(self.shape)

    def stride(self, i=None):
        return self._strides if i is None else self._strides[i]


def fwd_kvcache_paged(q, k_pages, v_pages, cache_seqlens, block_table, k_new=None, v_new=None, *, causal=False,
                      window_size=(-1, -1), scale=None, num_splits=0, out=None, lse=None, workspace=None,
                      alibi_slopes=None, softcap=0.0):
    """fwd_kvcache over a paged cache: returns (o, lse).

    k_pages, v_pages (num_pages, page_size, Hkv, d); block_table int32
    (B, pages_per_entry) on the device: row j of entry b is row j % page_size
    of page block_table[b, j // page_size].  The capacity of an entry is
    pages_per_entry * page_size.
    """
    _require_gpu(q, k_pages, v_pages, cache_seqlens, block_table)
    if k_new is not None:
        _require_gpu(k_new, v_new)
    lib = load_library()
    if k_pages.dim() != 4 or k_pages.shape != v_pages.shape:
        raise ValueError("k_pages and v_pages must be (num_pages, page_size, nheads_kv, headdim)")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != q.shape[0] \
            or block_table.stride(1) != 1:
        raise ValueError("block_table must be an int32 (batch, pages_per_entry) tensor with unit column stride")
    if cache_seqlens.dtype != torch.int32 or tuple(cache_seqlens.shape) != (q.shape[0],) \
            or not cache_seqlens.is_contiguous():
        raise ValueError("cache_seqlens must be a contiguous int32 tensor of shape (batch,)")
    num_pages, page_size = k_pages.shape[0], k_pages.shape[1]
    cap = block_table.shape[1] * page_size
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    # Parameters as for a contiguous cache of the entries' capacity, with the
    # pool's (page, row, head) strides in place of (batch, row, head).
    shape = (q.shape[0], cap, k_pages.shape[2], k_pages.shape[3])
    p = make_kv_params(q, _Layout(shape, k_pages.stride(), k_pages.dtype),
                       _Layout(shape, v_pages.stride(), v_pages.dtype), out, k_new, v_new, causal=causal,
                       window_size=window_size, scale=scale, num_splits=num_splits, alibi_slopes=alibi_slopes,
                       softcap=softcap)
    need = kvcache_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd_kvcache_paged(ctypes.byref(p), int(page_size), int(num_pages), _ptr(block_table),
                                        block_table.stride(0), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                        _ptr(cache_seqlens), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse),
                                        _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out, lse


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, window_size, scale, alibi_slopes, softcap):
        o, lse = fwd(q, k, v, causal=causal, window_size=window_size, scale=scale, alibi_slopes=alibi_slopes,
                     softcap=softcap)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (causal, window_size, scale, alibi_slopes, softcap)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        causal, window_size, scale, alibi_slopes, softcap = ctx.cfg
        do = do.contiguous() if do.stride() != o.stride() else do
        if do.stride() != o.stride():
            do = torch.empty_strided(o.shape, o.stride(), dtype=o.dtype, device=o.device).copy_(do)
        dq, dk, dv = bwd(do, q, k, v, o, lse, causal=causal, window_size=window_size, scale=scale,
                         alibi_slopes=alibi_slopes, softcap=softcap)
        return dq, dk, dv, None, None, None, None, None


def attention(q, k, v, *, causal=False, window_size=(-1, -1), scale=None, alibi_slopes=None, softcap=0.0):
    """Differentiable exact attention over (batch, seqlen, nheads, headdim) tensors."""
    return _Attention.apply(q, k, v, causal, tuple(window_size), scale, alibi_slopes, softcap)


class _AttentionVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_q, cu_k, max_q, max_k, causal, window_size, scale):
        o, lse = fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k, causal=causal, window_size=window_size, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse, cu_q, cu_k)
        ctx.cfg = (max_q, max_k, causal, window_size, scale)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, cu_q, cu_k = ctx.saved_tensors
        max_q, max_k, causal, window_size, scale = ctx.cfg
        if do.stride() != o.stride():
            do = torch.empty_strided(o.shape, o.stride(), dtype=o.dtype, device=o.device).copy_(do)
        dq, dk, dv = bwd_varlen(do, q, k, v, o, lse, cu_q, cu_k, max_q, max_k, causal=causal,
                                window_size=window_size, scale=scale)
        return dq, dk, dv, None, None, None, None, None, None, None


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
                     window_size=(-1, -1), scale=None):
    """Differentiable exact attention over a packed variable-length batch."""
    return _AttentionVarlen.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, int(max_seqlen_q), int(max_seqlen_k),
                                  causal, tuple(window_size), scale)


def _unpack_qkv(qkv):
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise ValueError("qkv must be (batch, seqlen, 3, nheads, headdim)")
    return qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]


class _AttentionQkvPacked(torch.autograd.Function):
    @staticmethod
    def forward(ctx, qkv, causal, window_size, scale):
        q, k, v = _unpack_qkv(qkv)
        o, lse = fwd(q, k, v, causal=causal, window_size=window_size, scale=scale)
        ctx.save_for_backward(qkv, o, lse)
        ctx.cfg = (causal, window_size, scale)
        return o

    @staticmethod
    def backward(ctx, do):
        qkv, o, lse = ctx.saved_tensors
        causal, window_size, scale = ctx.cfg
        q, k, v = _unpack_qkv(qkv)
        if do.stride() != o.stride():
            do = torch.empty_strided(o.shape, o.stride(), dtype=o.dtype, device=o.device).copy_(do)
        # The gradient is written straight into one packed tensor through
        # views with the strides of q, k and v.
        dqkv = torch.empty_like(qkv)
        dq, dk, dv = _unpack_qkv(dqkv)
        bwd(do, q, k, v, o, lse, causal=causal, window_size=window_size, scale=scale, dq=dq, dk=dk, dv=dv)
        return dqkv, None, None, None


def fwd_qkvpacked(qkv, *, causal=False, window_size=(-1, -1), scale=None, out=None, lse=None):
    """Forward of packed (batch, seqlen, 3, nheads, headdim) q/k/v: returns (o, lse)."""
    q, k, v = _unpack_qkv(qkv)
    return fwd(q, k, v, causal=causal, window_size=window_size, scale=scale, out=out, lse=lse)


def attention_qkvpacked(qkv, *, causal=False, window_size=(-1, -1), scale=None):
    """Differentiable attention over packed q/k/v; the gradient is packed the same way."""
    return _AttentionQkvPacked.apply(qkv, causal, tuple(window_size), scale)
