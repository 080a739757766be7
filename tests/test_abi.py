"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, the ctypes struct matches the C layout, and every invalid
argument is rejected on the host with the documented status before any device
call is made."""

import ctypes
import math
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

fa = pytest.importorskip("exact_tiled_attention_07_amd")
from exact_tiled_attention_07_amd import _native as N  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(N.LIB_PATH):
        pytest.skip("libfa.so not built")
    return N.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert header_functions() == sorted(
        ["fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_stage", "fa_bwd_workspace_size", "fa_fwd_kvcache",
         "fa_fwd_kvcache_paged",
         "fa_fwd_kvcache_workspace_size", "fa_fwd_varlen", "fa_bwd_varlen", "fa_bwd_varlen_workspace_size",
         "fa_status_string", "fa_last_error", "fa_version"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (fa_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)
        assert name in N.SIGNATURES


@pytest.mark.parametrize("cname,ctype", [("fa_params", N.FaParams), ("fa_kvcache_params", N.FaKvParams),
                                         ("fa_varlen_params", N.FaVarlenParams)])
def test_struct_layout_matches_c(tmp_path, cname, ctype):
    fields = [f for f, _ in ctype._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "fa.h"', "int main(void){",
           f'printf("%zu\\n", sizeof({cname}));']
    src += [f'printf("%zu\\n", offsetof({cname}, {f}));' for f in fields]
    src += ["return 0;}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(ctype)
    for f, off in zip(fields, vals[1:]):
        assert getattr(ctype, f).offset == off, f


def test_header_compiles_as_c_and_cpp(tmp_path):
    c = tmp_path / "use.c"
    c.write_text('#include "fa.h"\nint f(void){ return fa_version(); }\n')
    for comp, std in (("gcc", "-std=c99"), ("g++", "-std=c++11")):
        subprocess.run([comp, std, "-Wall", "-Werror", "-x", "c" if comp == "gcc" else "c++",
                        "-I", os.path.join(ROOT, "include"), "-c", str(c), "-o", str(tmp_path / "u.o")],
                       check=True)


def test_status_strings_and_version(lib):
    assert lib.fa_version() == 10000
    for s, name in ((0, b"FA_OK"), (1, b"FA_ERR_INVALID_ARG"), (2, b"FA_ERR_UNSUPPORTED"), (3, b"FA_ERR_HIP")):
        assert lib.fa_status_string(s) == name
    assert lib.fa_status_string(99) == b"FA_STATUS_UNKNOWN"


# Fake, 16-byte aligned "device" addresses: validation must reject the call
# before anything is dereferenced or any HIP function runs.
A, B_, C, O, L, W = (0x10000 * (i + 1) for i in range(6))


def params(**kw):
    p = N.FaParams()
    b, nq, nk, hq, hkv, d = 2, 64, 64, 4, 2, 64
    p.batch, p.seqlen_q, p.seqlen_k, p.nheads_q, p.nheads_kv, p.headdim = b, nq, nk, hq, hkv, d
    qs = (nq * hq * d, hq * d, d)
    ks = (nk * hkv * d, hkv * d, d)
    p.q_strides, p.o_strides = N._I64x3(*qs), N._I64x3(*qs)
    p.k_strides, p.v_strides = N._I64x3(*ks), N._I64x3(*ks)
    p.dtype, p.scale, p.causal = N.FA_BF16, 0.125, 0
    p.window_left = p.window_right = -1
    for k, v in kw.items():
        if k.endswith("_strides"):
            v = N._I64x3(*v)
        setattr(p, k, v)
    return p


def call_fwd(lib, p, q=A, k=B_, v=C, o=O, lse=L):
    pp = ctypes.byref(p) if p is not None else None
    return lib.fa_fwd(pp, q, k, v, o, lse, None)


def call_bwd(lib, p, ws=W, ws_bytes=1 << 30, dq=0x70000, dk=0x80000, dv=0x90000):
    return lib.fa_bwd(ctypes.byref(p), 0xA0000, A, B_, C, O, L, dq, dk, dv, ws, ws_bytes, None)


def call_stage(lib, p, stage, ws=W, ws_bytes=1 << 30, dq=0x70000, dk=0x80000, dv=0x90000):
    return lib.fa_bwd_stage(ctypes.byref(p), stage, 0xA0000, A, B_, C, O, L, dq, dk, dv, ws, ws_bytes, None)


STAGES = (N.FA_BWD_PREPARE, N.FA_BWD_DKDV, N.FA_BWD_DQ)


INVALID = [
    ("nheads not divisible", dict(nheads_q=6, nheads_kv=4)),
    ("negative batch", dict(batch=-1)),
    ("negative seqlen", dict(seqlen_k=-5)),
    ("zero heads", dict(nheads_kv=0)),
    ("zero headdim", dict(headdim=0)),
    ("bad dtype", dict(dtype=7)),
    ("zero scale", dict(scale=0.0)),
    ("negative scale", dict(scale=-1.0)),
    ("inf scale", dict(scale=math.inf)),
    ("nan scale", dict(scale=math.nan)),
    ("window below -1", dict(window_left=-2)),
    ("right window below -1", dict(window_right=-3)),
    ("causal not 0/1", dict(causal=2)),
    ("negative softcap", dict(softcap=-1.0)),
    ("nan softcap", dict(softcap=math.nan)),
    ("inf softcap", dict(softcap=math.inf)),
    ("negative alibi stride", dict(alibi_batch_stride=-1)),
    ("reserved_mod set", dict(reserved_mod=1)),
]
UNSUPPORTED = [
    ("bf16 headdim 136", dict(headdim=136, q_strides=(64 * 4 * 136, 4 * 136, 136),
                              o_strides=(64 * 4 * 136, 4 * 136, 136), k_strides=(64 * 2 * 136, 2 * 136, 136),
                              v_strides=(64 * 2 * 136, 2 * 136, 136))),
    ("fp16 headdim 256", dict(dtype=1, headdim=256, q_strides=(64 * 4 * 256, 4 * 256, 256),
                              o_strides=(64 * 4 * 256, 4 * 256, 256), k_strides=(64 * 2 * 256, 2 * 256, 256),
                              v_strides=(64 * 2 * 256, 2 * 256, 256))),
    ("bf16 headdim 60", dict(headdim=60)),
    ("fp32 headdim 6", dict(dtype=0, headdim=6)),
    ("fp32 headdim 132", dict(dtype=0, headdim=132)),
    ("stride not 16 bytes", dict(k_strides=(64 * 2 * 64, 2 * 64, 68))),
    ("negative stride", dict(q_strides=(-16, 256, 64))),
    ("zero sequence stride (expanded k)", dict(k_strides=(64 * 2 * 64, 0, 64))),
    ("sequence stride below headdim (q rows overlap)", dict(q_strides=(64 * 4 * 64, 32, 64))),
    ("sequence stride below headdim (o rows overlap)", dict(o_strides=(64 * 4 * 64, 56, 64))),
    ("sequence stride below headdim (v rows overlap)", dict(v_strides=(64 * 2 * 64, 8, 64))),
    ("huge seqlen", dict(seqlen_q=1 << 31, seqlen_k=1 << 31)),
    ("misaligned alibi slopes", dict(alibi_slopes=0x1002)),
]


@pytest.mark.parametrize("name,kw", INVALID, ids=[x[0] for x in INVALID])
def test_invalid_arguments(lib, name, kw):
    assert call_fwd(lib, params(**kw)) == N.FA_ERR_INVALID_ARG
    assert lib.fa_last_error() != b""
    assert call_bwd(lib, params(**kw)) == N.FA_ERR_INVALID_ARG
    for st in STAGES:
        assert call_stage(lib, params(**kw), st) == N.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("name,kw", UNSUPPORTED, ids=[x[0] for x in UNSUPPORTED])
def test_unsupported_arguments(lib, name, kw):
    assert call_fwd(lib, params(**kw)) == N.FA_ERR_UNSUPPORTED
    assert call_bwd(lib, params(**kw)) == N.FA_ERR_UNSUPPORTED
    for st in STAGES:
        assert call_stage(lib, params(**kw), st) == N.FA_ERR_UNSUPPORTED


def call_noalloc(lib, p, dq=0x70000, dk=0x80000, dv=0x90000):
    pp = ctypes.byref(p) if p is not None else None
    return lib.fa_bwd_noalloc(pp, 0xA0000, A, B_, C, O, L, dq, dk, dv, None)


def test_noalloc_validation(lib):
    # fa_bwd_noalloc validates exactly as fa_bwd (minus the workspace) and
    # rejects problems whose row statistics exceed its 16 MiB static scratch,
    # all before any device call.
    assert call_noalloc(lib, None) == N.FA_ERR_INVALID_ARG
    for _, kw in INVALID:
        assert call_noalloc(lib, params(**kw)) == N.FA_ERR_INVALID_ARG
    for _, kw in UNSUPPORTED:
        assert call_noalloc(lib, params(**kw)) == N.FA_ERR_UNSUPPORTED
    assert call_noalloc(lib, params(), dk=A) == N.FA_ERR_INVALID_ARG  # aliases q
    # 2^21 rows of statistics fit exactly; one more 128-row block does not.
    fits = params(batch=1, seqlen_q=32768, seqlen_k=64, nheads_q=64, nheads_kv=2,
                  q_strides=(32768 * 64 * 64, 64 * 64, 64), o_strides=(32768 * 64 * 64, 64 * 64, 64))
    big = params(batch=1, seqlen_q=32769, seqlen_k=64, nheads_q=64, nheads_kv=2,
                 q_strides=(32769 * 64 * 64, 64 * 64, 64), o_strides=(32769 * 64 * 64, 64 * 64, 64))
    assert call_noalloc(lib, big) == N.FA_ERR_UNSUPPORTED
    assert b"static scratch" in lib.fa_last_error()
    assert call_noalloc(lib, fits) == N.FA_ERR_HIP  # valid: reaches the device check (no GPU here)
    assert call_noalloc(lib, params(batch=0)) == N.FA_OK


def test_backward_stage_validation(lib):
    # Unknown stages are rejected; every stage checks every pointer and the
    # workspace exactly as fa_bwd does.
    for bad in (-1, 3, 1 << 20):
        assert call_stage(lib, params(), bad) == N.FA_ERR_INVALID_ARG
        assert b"stage" in lib.fa_last_error()
    p = params()
    n = ctypes.c_size_t()
    assert lib.fa_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == N.FA_OK
    for st in STAGES:
        assert call_stage(lib, p, st, dq=None) == N.FA_ERR_INVALID_ARG
        assert call_stage(lib, p, st, dk=A) == N.FA_ERR_INVALID_ARG
        assert call_stage(lib, p, st, ws_bytes=n.value - 4) == N.FA_ERR_INVALID_ARG
        assert b"workspace" in lib.fa_last_error()
        pe = params(batch=0)
        assert lib.fa_bwd_stage(ctypes.byref(pe), st, None, None, None, None, None, None, None, None, None,
                                None, 0, None) == N.FA_OK


def test_null_and_misaligned_pointers(lib):
    assert call_fwd(lib, None) == N.FA_ERR_INVALID_ARG
    assert b"params" in lib.fa_last_error()
    assert call_fwd(lib, params(), q=None) == N.FA_ERR_INVALID_ARG
    assert call_fwd(lib, params(), lse=None) == N.FA_ERR_INVALID_ARG
    assert call_fwd(lib, params(), v=C + 8) == N.FA_ERR_UNSUPPORTED
    assert call_fwd(lib, params(), o=A) == N.FA_ERR_INVALID_ARG  # o aliases q
    assert call_bwd(lib, params(), dq=None) == N.FA_ERR_INVALID_ARG
    assert call_bwd(lib, params(), dk=A) == N.FA_ERR_INVALID_ARG  # dk aliases q


def test_workspace_size_and_check(lib):
    p = params()
    n = ctypes.c_size_t()
    assert lib.fa_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == N.FA_OK
    # two float32 arrays of batch * nheads_q * (seqlen_q rounded up to 128)
    assert n.value == ((2 * 4 * 2 * 4 * 128 + 255) // 256) * 256
    assert lib.fa_bwd_workspace_size(ctypes.byref(p), None) == N.FA_ERR_INVALID_ARG
    assert call_bwd(lib, p, ws_bytes=n.value - 4) == N.FA_ERR_INVALID_ARG
    assert b"workspace" in lib.fa_last_error()
    assert call_bwd(lib, p, ws=None) == N.FA_ERR_INVALID_ARG


def test_empty_problems_return_ok_without_device(lib):
    # Nothing to compute: OK with NULL pointers and no device access.
    assert call_fwd(lib, params(batch=0), q=None, k=None, v=None, o=None, lse=None) == N.FA_OK
    assert call_fwd(lib, params(seqlen_q=0), q=None, o=None, lse=None, k=None, v=None) == N.FA_OK
    p = params(batch=0)
    assert lib.fa_bwd(ctypes.byref(p), None, None, None, None, None, None, None, None, None, None, 0,
                      None) == N.FA_OK


def test_error_message_is_per_thread(lib):
    import threading
    call_fwd(lib, params(nheads_q=3))
    main_msg = lib.fa_last_error()
    seen = []

    def worker():
        seen.append(lib.fa_last_error())
        call_fwd(lib, params(scale=-1.0))
        seen.append(lib.fa_last_error())

    t = threading.Thread(target=worker)
    t.start()
    t.join()
    assert seen[0] == b""
    assert b"scale" in seen[1]
    assert lib.fa_last_error() == main_msg and b"multiple" in main_msg


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU error path")
def test_valid_call_without_gpu_reports_hip_error(lib):
    # Validation passes, so the library asks HIP for the device and must fail
    # cleanly (no kernel is ever launched without a device).
    assert call_fwd(lib, params()) == N.FA_ERR_HIP
    assert b"hip" in lib.fa_last_error().lower()
    for st in STAGES:
        assert call_stage(lib, params(), st) == N.FA_ERR_HIP


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd(q, q, q)


def _struct_bytes(p):
    return bytes(memoryview(p).cast("B"))


def test_memoised_params_match_fresh_params():
    """fwd/bwd reuse the FaParams of an earlier call with the same shapes,
    strides, dtypes and options; the reused struct must be byte-identical to
    a fresh make_params, and any change in those inputs must build a new one."""
    import torch
    N._PARAMS_CACHE.clear()
    q = torch.zeros(2, 8, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(2, 16, 2, 64, dtype=torch.bfloat16)
    base = dict(causal=True, window_size=(-1, -1), scale=None, softcap=0.0)
    variants = [
        (q, k, k, q, base),
        (q, k, k, q, dict(base, causal=False)),
        (q, k, k, q, dict(base, window_size=(3, 0))),
        (q, k, k, q, dict(base, window_size=[3, 0])),
        (q, k, k, q, dict(base, scale=0.5)),
        (q, k, k, q, dict(base, softcap=30.0)),
        (q.transpose(1, 2).contiguous().transpose(1, 2), k, k, q, base),
        (q, k[:, :8], k[:, :8], q, base),
        (q.half(), k.half(), k.half(), q.half(), base),
    ]
    seen = {}
    for qq, kk, vv, oo, kw in variants:
        first = N._dense_params(qq, kk, vv, oo, kw["causal"], kw["window_size"], kw["scale"], None, kw["softcap"])
        again = N._dense_params(qq, kk, vv, oo, kw["causal"], kw["window_size"], kw["scale"], None, kw["softcap"])
        assert again is first
        fresh = N.make_params(qq, kk, vv, oo, **kw)
        assert _struct_bytes(first[0]) == _struct_bytes(fresh)
        seen.setdefault(_struct_bytes(fresh), set()).add(id(first[0]))
    # one cached struct per distinct parameter set (the list and tuple windows share one)
    assert len(seen) == len(variants) - 1
    assert all(len(ids) == 1 for ids in seen.values())
    # a call with ALiBi slopes carries a pointer and is never served from the cache
    slopes = torch.zeros(4, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        N._dense_params(q, k, k, q, True, (-1, -1), None, slopes, 0.0)
    # invalid layouts are still rejected, cached or not
    with pytest.raises(ValueError, match="headdim"):
        strided_d = torch.zeros(2, 8, 64, 4, dtype=torch.bfloat16).transpose(2, 3)
        N._dense_params(strided_d, k, k, q, True, (-1, -1), None, None, 0.0)
    N._PARAMS_CACHE.clear()


def test_missing_library_fails_loudly(tmp_path):
    code = ("import exact_tiled_attention_07_amd._native as N; N.LIB_PATH = '/nonexistent/libfa.so'\n"
            "try:\n    N.load_library()\nexcept RuntimeError as e:\n    print('RAISED', 'missing' in str(e))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "RAISED True" in out.stdout, out.stderr


def test_library_has_no_undefined_kernel_symbols(lib):
    # Every kernel launcher's host stub must be defined in the library itself.
    out = subprocess.run(["nm", "-D", "--undefined-only", N.LIB_PATH], capture_output=True, text=True).stdout
    missing = [l for l in out.splitlines() if "_ZN2fa" in l]
    assert not missing, missing


# --------------------------------------------------------------------------
# fa_fwd_kvcache: host-side validation, workspace size, part count.
# --------------------------------------------------------------------------
KQ, KK, KV_, KN, VN, KO, KL, KS, KW = (0x100000 * (i + 1) for i in range(9))


def kv_params(num_splits=0, **kw):
    """B=2, Nq=1, Hq=4, Hkv=2, d=64, capacity 256, contiguous caches."""
    base = dict(seqlen_q=1, seqlen_k=256, q_strides=(1 * 4 * 64, 4 * 64, 64), o_strides=(1 * 4 * 64, 4 * 64, 64),
                k_strides=(256 * 2 * 64, 2 * 64, 64), v_strides=(256 * 2 * 64, 2 * 64, 64))
    base.update({k: v for k, v in kw.items() if not k.startswith(("knew", "vnew")) and k != "reserved"})
    p = N.FaKvParams()
    p.base = params(**base)
    p.knew_strides = N._I64x3(*kw.get("knew_strides", (1 * 2 * 64, 2 * 64, 64)))
    p.vnew_strides = N._I64x3(*kw.get("vnew_strides", (1 * 2 * 64, 2 * 64, 64)))
    p.num_splits = num_splits
    p.reserved = kw.get("reserved", 0)
    return p


def kv_ws(lib, p):
    n = ctypes.c_size_t()
    st = lib.fa_fwd_kvcache_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def call_kv(lib, p, q=KQ, kc=KK, vc=KV_, lens=KS, kn=KN, vn=VN, o=KO, lse=KL, ws=KW, ws_bytes=1 << 30):
    pp = ctypes.byref(p) if p is not None else None
    return lib.fa_fwd_kvcache(pp, q, kc, vc, lens, kn, vn, o, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("name,kw", INVALID, ids=[x[0] for x in INVALID])
def test_kvcache_invalid_arguments(lib, name, kw):
    assert call_kv(lib, kv_params(**kw)) == N.FA_ERR_INVALID_ARG
    assert kv_ws(lib, kv_params(**kw))[0] == N.FA_ERR_INVALID_ARG


def test_kvcache_specific_validation(lib):
    assert call_kv(lib, None) == N.FA_ERR_INVALID_ARG
    assert call_kv(lib, kv_params(num_splits=-1)) == N.FA_ERR_INVALID_ARG
    assert b"num_splits" in lib.fa_last_error()
    assert call_kv(lib, kv_params(reserved=1)) == N.FA_ERR_INVALID_ARG
    # without new rows their strides are not looked at (here: zeros, Nq = 4)
    nq4 = dict(seqlen_q=4, q_strides=(4 * 4 * 64, 4 * 64, 64), o_strides=(4 * 4 * 64, 4 * 64, 64),
               knew_strides=(0, 0, 0), vnew_strides=(0, 0, 0))
    assert call_kv(lib, kv_params(**nq4), kn=None, vn=None) != N.FA_ERR_UNSUPPORTED
    assert call_kv(lib, kv_params(**nq4)) == N.FA_ERR_UNSUPPORTED
    assert call_kv(lib, kv_params(), kn=None) == N.FA_ERR_INVALID_ARG       # one of the pair
    assert b"k_new" in lib.fa_last_error()
    assert call_kv(lib, kv_params(), lens=None) == N.FA_ERR_INVALID_ARG
    assert call_kv(lib, kv_params(), lens=KS + 2) == N.FA_ERR_UNSUPPORTED   # int32 array misaligned
    assert call_kv(lib, kv_params(), q=None) == N.FA_ERR_INVALID_ARG
    assert call_kv(lib, kv_params(), kc=KK + 8) == N.FA_ERR_UNSUPPORTED
    assert call_kv(lib, kv_params(), o=KQ) == N.FA_ERR_INVALID_ARG          # o aliases q
    assert call_kv(lib, kv_params(), lse=KN) == N.FA_ERR_INVALID_ARG        # lse aliases k_new
    assert call_kv(lib, kv_params(), ws=None) == N.FA_ERR_INVALID_ARG
    st, need = kv_ws(lib, kv_params())
    assert st == N.FA_OK
    assert call_kv(lib, kv_params(), ws_bytes=need - 4) == N.FA_ERR_INVALID_ARG
    assert b"workspace" in lib.fa_last_error()
    assert lib.fa_fwd_kvcache_workspace_size(ctypes.byref(kv_params()), None) == N.FA_ERR_INVALID_ARG


KV_UNSUPPORTED = [
    ("fp32", dict(dtype=0)),
    ("headdim 144", dict(headdim=144, q_strides=(4 * 144, 4 * 144, 144), o_strides=(4 * 144, 4 * 144, 144),
                         k_strides=(256 * 2 * 144, 2 * 144, 144), v_strides=(256 * 2 * 144, 2 * 144, 144),
                         knew_strides=(2 * 144, 2 * 144, 144), vnew_strides=(2 * 144, 2 * 144, 144))),
    ("new-row stride not 16 bytes", dict(knew_strides=(2 * 64, 2 * 64, 60))),
    ("negative new-row stride", dict(vnew_strides=(-128, 128, 64))),
    ("overlapping new rows", dict(seqlen_q=4, q_strides=(4 * 4 * 64, 4 * 64, 64), o_strides=(4 * 4 * 64, 4 * 64, 64),
                                  knew_strides=(4 * 2 * 64, 32, 64), vnew_strides=(4 * 2 * 64, 2 * 64, 64))),
    ("overlapping cache rows", dict(k_strides=(256 * 2 * 64, 0, 64))),
]


@pytest.mark.parametrize("name,kw", KV_UNSUPPORTED, ids=[x[0] for x in KV_UNSUPPORTED])
def test_kvcache_unsupported_arguments(lib, name, kw):
    assert call_kv(lib, kv_params(**kw)) == N.FA_ERR_UNSUPPORTED


def test_kvcache_workspace_size_and_parts(lib):
    # B * Hq * Nq rows, each with parts * (d + 1) floats; parts = num_splits
    # when given (capped by the 32-key tiles of the capacity).
    for splits, parts in ((1, 1), (3, 3), (8, 8), (100, 8)):
        st, n = kv_ws(lib, kv_params(num_splits=splits))
        assert st == N.FA_OK
        assert n == ((2 * 4 * 1 * parts * 65 * 4 + 255) // 256) * 256, (splits, n)
    # num_splits = 0: the library's choice, at least one part and at most a
    # part per four key tiles (256 keys: 8 tiles -> 2 parts).
    st, n = kv_ws(lib, kv_params())
    assert st == N.FA_OK and n == ((2 * 4 * 2 * 65 * 4 + 255) // 256) * 256
    # Longer caches get more parts when the batch is small.
    st, n_long = kv_ws(lib, kv_params(seqlen_k=65536, k_strides=(65536 * 128, 128, 64),
                                      v_strides=(65536 * 128, 128, 64)))
    assert st == N.FA_OK and n_long > n


def test_kvcache_empty_problems_return_ok_without_device(lib):
    assert call_kv(lib, kv_params(batch=0), q=None, kc=None, vc=None, lens=None, kn=None, vn=None, o=None,
                   lse=None, ws=None, ws_bytes=0) == N.FA_OK
    assert call_kv(lib, kv_params(seqlen_q=0), q=None, kc=None, vc=None, lens=None, kn=None, vn=None, o=None,
                   lse=None, ws=None, ws_bytes=0) == N.FA_OK


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU error path")
def test_kvcache_valid_call_without_gpu_reports_hip_error(lib):
    assert call_kv(lib, kv_params()) == N.FA_ERR_HIP
    assert call_kv(lib, kv_params(), kn=None, vn=None) == N.FA_ERR_HIP
    # An empty cache with no append needs no cache pointers.
    p = kv_params(seqlen_k=0)
    assert call_kv(lib, p, kc=None, vc=None, kn=None, vn=None) == N.FA_ERR_HIP


def test_python_kvcache_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 2, 64, dtype=torch.bfloat16)
    c = torch.zeros(1, 32, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd_kvcache(q, c, c, torch.zeros(1, dtype=torch.int32))


# --------------------------------------------------------------------------
# fa_fwd_varlen / fa_bwd_varlen: host-side validation and workspace size.
# --------------------------------------------------------------------------
CQ, CK = 0x300000, 0x310000


def vl_params(total_q=100, total_k=120, **kw):
    """3 packed sequences, Hq=4, Hkv=2, d=64, max lengths 64; strides[0] deliberately garbage."""
    base = dict(batch=3, q_strides=(12345, 4 * 64, 64), o_strides=(7, 4 * 64, 64), k_strides=(3, 2 * 64, 64),
                v_strides=(1, 2 * 64, 64))
    base.update(kw)
    p = N.FaVarlenParams()
    p.base = params(**base)
    p.total_q, p.total_k = total_q, total_k
    return p


def call_fwd_vl(lib, p, q=A, k=B_, v=C, cq=CQ, ck=CK, o=O, lse=L):
    pp = ctypes.byref(p) if p is not None else None
    return lib.fa_fwd_varlen(pp, q, k, v, cq, ck, o, lse, None)


def call_bwd_vl(lib, p, ws=W, ws_bytes=1 << 30, cq=CQ, ck=CK, dq=0x70000, dk=0x80000, dv=0x90000):
    return lib.fa_bwd_varlen(ctypes.byref(p), 0xA0000, A, B_, C, O, L, cq, ck, dq, dk, dv, ws, ws_bytes, None)


@pytest.mark.parametrize("name,kw", INVALID, ids=[x[0] for x in INVALID])
def test_varlen_invalid_arguments(lib, name, kw):
    assert call_fwd_vl(lib, vl_params(**kw)) == N.FA_ERR_INVALID_ARG
    assert call_bwd_vl(lib, vl_params(**kw)) == N.FA_ERR_INVALID_ARG


def test_varlen_specific_validation(lib):
    assert call_fwd_vl(lib, None) == N.FA_ERR_INVALID_ARG
    assert call_fwd_vl(lib, vl_params(total_q=-1)) == N.FA_ERR_INVALID_ARG
    assert call_fwd_vl(lib, vl_params(total_k=1 << 31)) == N.FA_ERR_UNSUPPORTED
    assert call_fwd_vl(lib, vl_params(), cq=None) == N.FA_ERR_INVALID_ARG
    assert b"cu_seqlens_q" in lib.fa_last_error()
    assert call_fwd_vl(lib, vl_params(), ck=CK + 2) == N.FA_ERR_UNSUPPORTED
    assert call_fwd_vl(lib, vl_params(), o=A) == N.FA_ERR_INVALID_ARG
    assert call_bwd_vl(lib, vl_params(), cq=None) == N.FA_ERR_INVALID_ARG
    assert call_bwd_vl(lib, vl_params(), dk=A) == N.FA_ERR_INVALID_ARG
    # strides[0] is ignored: the garbage batch strides above are accepted,
    # while a bad row stride is not.
    assert call_fwd_vl(lib, vl_params(k_strides=(0, 2 * 64, 68))) == N.FA_ERR_UNSUPPORTED


def test_varlen_workspace_size(lib):
    p = vl_params()
    n = ctypes.c_size_t()
    assert lib.fa_bwd_varlen_workspace_size(ctypes.byref(p), ctypes.byref(n)) == N.FA_OK
    # two float32 arrays of nheads_q * (total_q + 128 * batch)
    assert n.value == ((2 * 4 * (100 + 128 * 3) * 4 + 255) // 256) * 256
    assert lib.fa_bwd_varlen_workspace_size(ctypes.byref(p), None) == N.FA_ERR_INVALID_ARG
    assert call_bwd_vl(lib, p, ws_bytes=n.value - 4) == N.FA_ERR_INVALID_ARG
    assert b"workspace" in lib.fa_last_error()


def test_varlen_empty_problems_return_ok_without_device(lib):
    p = vl_params(total_q=0, total_k=0)
    assert call_fwd_vl(lib, p, q=None, k=None, v=None, cq=None, ck=None, o=None, lse=None) == N.FA_OK
    assert lib.fa_bwd_varlen(ctypes.byref(vl_params(batch=0, total_q=0, total_k=0)), None, None, None, None,
                             None, None, None, None, None, None, None, W, 1 << 20, None) == N.FA_OK


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU error path")
def test_varlen_valid_call_without_gpu_reports_hip_error(lib):
    assert call_fwd_vl(lib, vl_params()) == N.FA_ERR_HIP
    assert call_bwd_vl(lib, vl_params()) == N.FA_ERR_HIP


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU error path")
def test_valid_modifiers_pass_validation(lib):
    # Slopes (aligned, per batch entry) and a softcap are accepted: the call
    # gets as far as the device check.
    p = params(alibi_slopes=0x1000, alibi_batch_stride=4, softcap=30.0)
    assert call_fwd(lib, p) == N.FA_ERR_HIP
    assert call_bwd(lib, p) == N.FA_ERR_HIP


def test_python_binding_checks_slope_shape():
    import torch
    q = torch.zeros(2, 8, 4, 64, dtype=torch.bfloat16)
    p = N.FaParams()
    with pytest.raises(ValueError, match="alibi_slopes"):
        N._set_modifiers(p, 4, 2, torch.zeros(3, dtype=torch.float32), 0.0)
    with pytest.raises(ValueError, match="alibi_slopes"):
        N._set_modifiers(p, 4, 2, torch.zeros(4, dtype=torch.float64), 0.0)
    del q


# --------------------------------------------------------------------------
# fa_fwd_kvcache_paged: paging arguments.
# --------------------------------------------------------------------------
BT = 0x320000


def call_paged(lib, p, page_size=64, num_pages=16, bt=BT, bt_stride=4, **kw):
    a = dict(q=KQ, kc=KK, vc=KV_, lens=KS, kn=KN, vn=VN, o=KO, lse=KL, ws=KW, ws_bytes=1 << 30)
    a.update(kw)
    return lib.fa_fwd_kvcache_paged(ctypes.byref(p), page_size, num_pages, bt, bt_stride, a["q"], a["kc"], a["vc"],
                                    a["lens"], a["kn"], a["vn"], a["o"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_paged_kvcache_validation(lib):
    p = kv_params()  # capacity 256 = 4 pages of 64
    for bad in (dict(page_size=0), dict(page_size=48), dict(page_size=-64), dict(page_size=512),
                dict(num_pages=0), dict(bt_stride=3), dict(bt=None)):
        assert call_paged(lib, p, **bad) == N.FA_ERR_INVALID_ARG, bad
    assert call_paged(lib, p, bt=BT + 2) == N.FA_ERR_UNSUPPORTED
    # the contiguous checks still apply
    assert call_paged(lib, kv_params(num_splits=-1)) == N.FA_ERR_INVALID_ARG
    assert call_paged(lib, p, lens=None) == N.FA_ERR_INVALID_ARG
    assert call_paged(lib, kv_params(batch=0), q=None, kc=None, vc=None, lens=None, kn=None, vn=None, o=None,
                      lse=None, ws=None, ws_bytes=0) == N.FA_OK


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU error path")
def test_paged_kvcache_valid_call_without_gpu_reports_hip_error(lib):
    assert call_paged(lib, kv_params()) == N.FA_ERR_HIP
    assert call_paged(lib, kv_params(), page_size=256, bt_stride=1) == N.FA_ERR_HIP


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU error path")
@pytest.mark.parametrize("d", [8, 32, 40, 96, 120])
def test_head_dims_multiple_of_8_pass_validation(lib, d):
    kw = dict(headdim=d, q_strides=(64 * 4 * d, 4 * d, d), o_strides=(64 * 4 * d, 4 * d, d),
              k_strides=(64 * 2 * d, 2 * d, d), v_strides=(64 * 2 * d, 2 * d, d))
    for dt in (N.FA_F16, N.FA_BF16):
        assert call_fwd(lib, params(dtype=dt, **kw)) == N.FA_ERR_HIP
        assert call_bwd(lib, params(dtype=dt, **kw)) == N.FA_ERR_HIP


def test_plain_c_caller_builds_and_links(tmp_path, lib):
    # tests/c_caller/fa_c_caller.c uses only include/fa.h and the HIP runtime;
    # it must compile as C99 and link against the library (run on a GPU in
    # tests/test_c_caller_gpu.py).
    import shutil
    if shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are not available")
    exe = tmp_path / "fa_c_caller"
    libdir = os.path.dirname(N.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_caller", "fa_c_caller.c"),
                    "-o", str(exe), "-L", libdir, "-lfa", "-L", "/opt/rocm/lib", "-lamdhip64", "-lm",
                    f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 1 and "usage" in out.stderr
