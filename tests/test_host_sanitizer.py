"""The C ABI's host code built with the address and undefined-behaviour
sanitizers (and -Werror), replaying the validation matrix of test_abi.py.

fa_api.cpp (every check the ABI makes before it touches the device) is compiled
for the host with ASan and UBSan; the kernel launchers are replaced by stubs
that report the launch as unavailable, so no device code is built and no GPU is
needed.  A small C++ driver reads the matrix -- the same parameter structs the
ctypes tests pass, as raw bytes -- calls each entry point with fake, aligned
pointers and checks the status.  Any sanitizer report aborts the driver.
"""

import os
import shutil
import subprocess

import pytest

import test_abi as T
from exact_tiled_attention_07_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_07_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
# Host-only sanitizers: on a hipcc line every -fsanitize= is preceded by
# -Xarch_host, so no device code is ever built with them.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
WARN = ["-Wall", "-Werror"]


def _tools():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("ROCm compilers not available")
    return hipcc, clangxx


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{err}\n{res.stdout}"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    hipcc, clangxx = _tools()
    out = tmp_path_factory.mktemp("host_sanitizer")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "fa_api.cpp"), os.path.join(SAN, "launch_stubs.hip")):
        obj = str(out / (os.path.basename(src) + ".o"))
        _run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *WARN, *HOST_SAN, *inc,
              "-c", src, "-o", obj])
        objs.append(obj)
    obj = str(out / "abi_driver.o")
    _run([clangxx, "-O1", "-g", "-std=c++17", *WARN, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          *inc, "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", obj])
    objs.append(obj)
    exe = str(out / "abi_driver")
    _run([clangxx, "-fsanitize=address,undefined", *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    return exe


def _matrix():
    lines = []

    def add(entry, status, struct):
        lines.append(f"{entry} {int(status)} {bytes(struct).hex()}")

    for _, kw in T.INVALID:
        for e in ("fwd", "bwd", "bwd_ws", "stage0", "stage1", "stage2", "bwd_na"):
            add(e, N.FA_ERR_INVALID_ARG, T.params(**kw))
        add("kv", N.FA_ERR_INVALID_ARG, T.kv_params(**kw))
        add("kv_ws", N.FA_ERR_INVALID_ARG, T.kv_params(**kw))
        add("vl_fwd", N.FA_ERR_INVALID_ARG, T.vl_params(**kw))
        add("vl_bwd", N.FA_ERR_INVALID_ARG, T.vl_params(**kw))
    for _, kw in T.UNSUPPORTED:
        for e in ("fwd", "bwd", "stage0", "stage1", "stage2", "bwd_na"):
            add(e, N.FA_ERR_UNSUPPORTED, T.params(**kw))
    for _, kw in T.KV_UNSUPPORTED:
        add("kv", N.FA_ERR_UNSUPPORTED, T.kv_params(**kw))
    add("kv", N.FA_ERR_INVALID_ARG, T.kv_params(num_splits=-1))
    add("vl_fwd", N.FA_ERR_INVALID_ARG, T.vl_params(total_q=-1))
    add("vl_fwd", N.FA_ERR_UNSUPPORTED, T.vl_params(total_k=1 << 31))
    add("vl_fwd", N.FA_ERR_UNSUPPORTED, T.vl_params(k_strides=(0, 2 * 64, 68)))
    # Valid calls pass every check and reach the device check or a launcher
    # stub: FA_ERR_HIP either way; the size queries succeed.
    for e in ("fwd", "bwd", "stage0", "stage1", "stage2", "bwd_na"):
        add(e, N.FA_ERR_HIP, T.params())
    add("bwd_na", N.FA_ERR_UNSUPPORTED, T.params(batch=1, seqlen_q=32769, seqlen_k=64, nheads_q=64, nheads_kv=2,
                                                 q_strides=(32769 * 64 * 64, 64 * 64, 64),
                                                 o_strides=(32769 * 64 * 64, 64 * 64, 64)))
    add("bwd_ws", N.FA_OK, T.params())
    add("kv", N.FA_ERR_HIP, T.kv_params())
    add("kv_ws", N.FA_OK, T.kv_params())
    add("vl_fwd", N.FA_ERR_HIP, T.vl_params())
    add("vl_bwd", N.FA_ERR_HIP, T.vl_params())
    add("vl_ws", N.FA_OK, T.vl_params())
    # Empty problems return FA_OK before any device call.
    add("fwd", N.FA_OK, T.params(batch=0))
    add("bwd", N.FA_OK, T.params(seqlen_q=0, seqlen_k=0))
    return lines


def test_validation_matrix_under_sanitizers(driver):
    lines = _matrix()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    res = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                         timeout=300)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert f"{len(lines)} cases, 0 mismatches" in res.stdout, res.stdout


def test_sanitizer_is_live(driver, tmp_path):
    # The build really is instrumented: the address sanitizer's runtime is linked in.
    nm = shutil.which("nm")
    if not nm:
        pytest.skip("nm not available")
    syms = subprocess.run([nm, driver], capture_output=True, text=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle" in syms
