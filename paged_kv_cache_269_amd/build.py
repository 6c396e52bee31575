"""Build libpagedattn.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libpagedattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "api_blocks.cpp", "block_manager.cpp", "reshape_and_cache.hip", "copy_blocks.hip",
           "decode_valu.hip", "decode_mfma.hip", "prefix.hip", "multi_query.hip",
           "reduce.hip", "decode_static.hip"]

# Packed fp32 ALU ops are kept out of the generated code.  Matrix-core
# accumulators are kept in ordinary VGPRs: the online-softmax rescale works on
# them with vector ALU ops, which cannot read accumulation registers.
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1",
                "-Wall", "-I", os.path.join(ROOT, "include")]


def _compile(src: str, extra, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(extra_flags=(), jobs: int = 8, lib_path: str = LIB_PATH) -> str:
    """Compile every kernel source and link the library (libpagedattn.so in
    the package by default); returns its path.  ``extra_flags`` reach every
    hipcc compile (e.g. -D tuning macros of the kernels)."""
    build_dir = BUILD_DIR if lib_path == LIB_PATH else lib_path + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags), build_dir), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build())
