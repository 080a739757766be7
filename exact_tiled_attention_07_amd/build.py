"""Build the HIP library libfa.so for gfx950 (in-tree, next to this file).

    python -m exact_tiled_attention_07_amd.build

Every HIP source is compiled with hipcc for --offload-arch=gfx950; the C ABI
layer (fa_api.cpp) is compiled as HIP host code.  Objects go to _build/ at the
repository root; the shared library goes into the package directory so that it
travels with the source tree.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

SOURCES = ["fa_api.cpp", "fwd_mfma.hip", "bwd_mfma.hip", "f32_valu.hip", "decode.hip"]
HEADERS = ["common.hpp", "tile_io.hpp", "launch.hpp"]

ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Werror",
    # Packed-fp32 VALU forms stay off: hipcc -O3 would otherwise fuse pairs of
    # fp32 adds/muls/FMAs into them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


# Per-source extra compiler flags.
SOURCE_FLAGS = {}


def _compile(src, build_dir=BUILD_DIR, defines=(), extra=None):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    flags = list(SOURCE_FLAGS.get(src, ())) + list((extra or {}).get(src, ()))
    cmd = [hipcc(), *COMMON_FLAGS, *flags, *[f"-D{d}" for d in defines], "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj, err


def build(verbose=True, lib_path=LIB_PATH, build_dir=BUILD_DIR, defines=(), extra_flags=None):
    """Compile every source and link libfa.so; returns the library path.
    ``defines`` (NAME=VALUE strings) override the kernels' launch configuration;
    ``extra_flags`` maps a source file name to additional compiler flags."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda src: _compile(src, build_dir, defines, extra_flags), SOURCES))
    for _, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build()
