"""The C ABI used from plain C: tests/c_caller/fa_c_caller.c allocates device
memory with the HIP runtime, calls fa_fwd and fa_bwd, and writes the results;
they are compared with the float64 oracle.  No torch and no Python binding on
the library's side of the boundary."""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import exact_tiled_attention_07_amd as fa  # noqa: E402
import oracle  # noqa: E402
from exact_tiled_attention_07_amd.workloads import random_qkv  # noqa: E402
from gpu_util import TOL, f64  # noqa: E402
from compare import within  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _build(tmp):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = os.path.join(tmp, "fa_c_caller")
    libdir = os.path.dirname(fa.library_path())
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_caller", "fa_c_caller.c"), "-o", exe,
           "-L", libdir, "-lfa", "-L", "/opt/rocm/lib", "-lamdhip64", "-lm", f"-Wl,-rpath,{libdir}",
           "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _bf16_file(path, t):
    t.contiguous().view(torch.int16).numpy().tofile(path)


def _read_bf16(path, shape):
    raw = np.fromfile(path, dtype=np.uint16).astype(np.uint32) << 16
    return raw.view(np.float32).astype(np.float64).reshape(shape)


@pytest.mark.parametrize("shape,causal", [((2, 200, 8, 2, 128), 1), ((1, 77, 4, 4, 64), 0), ((2, 130, 4, 1, 96), 1)])
def test_plain_c_caller_matches_oracle(tmp_path, shape, causal):
    b, n, hq, hkv, d = shape
    exe = _build(str(tmp_path))
    q, k, v, do = random_qkv((b, n, hq, d), (b, n, hkv, d), "bf16", seed=1500 + n)
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _bf16_file(str(tmp_path / f"{name}.bin"), t)
    run = subprocess.run([exe, str(tmp_path), str(b), str(n), str(hq), str(hkv), str(d), str(causal)],
                         capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    o = _read_bf16(str(tmp_path / "o.bin"), (b, n, hq, d))
    lse = np.fromfile(str(tmp_path / "lse.bin"), dtype=np.float32).astype(np.float64).reshape(b, hq, n)
    dq = _read_bf16(str(tmp_path / "dq.bin"), (b, n, hq, d))
    dk = _read_bf16(str(tmp_path / "dk.bin"), (b, n, hkv, d))
    dv = _read_bf16(str(tmp_path / "dv.bin"), (b, n, hkv, d))
    o_ref, lse_ref = oracle.attention_fwd(f64(q), f64(k), f64(v), causal=bool(causal))
    g_ref = oracle.attention_bwd(f64(do), f64(q), f64(k), f64(v), causal=bool(causal))
    tol = TOL[torch.bfloat16]
    for name, got, ref, dt, t in (("O", o, o_ref, "bf16", tol), ("LSE", lse, lse_ref, "fp32", tol),
                                  ("dq", dq, g_ref[0], "bf16", 2 * tol), ("dk", dk, g_ref[1], "bf16", 2 * tol),
                                  ("dv", dv, g_ref[2], "bf16", 2 * tol)):
        ok, info = within(got, ref, dt, t)
        assert ok, f"{name}: {info}"
