"""Build the HIP library libkvtier.so for gfx950, in-tree.

    python -m tiered_int2_fp16_amd.build

Every HIP source is compiled for gfx950 with packed FP32 instructions
disabled; objects go to ``_build/`` and the shared library to ``_lib/``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(OUT_DIR, "libkvtier.so")

SOURCES = ["api.hip", "attn.hip", "route.hip", "transitions.hip", "prefill_scores.hip", "probe.hip",
           "host_core.cpp"]
ARCH = os.environ.get("KVTIER_ARCH", "gfx950")


# Sources whose kernels take leading scalar arguments meant to be preloaded
# (attn_kernel: page table, token counts, row length, query, query heads,
# head group).
KERNARG_PRELOAD = {"attn.hip": 6}


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [hipcc()] + _flags() + ["-c", path, "-o", obj]
    if src in KERNARG_PRELOAD:
        # the first N kernel arguments of every kernel in the file arrive in SGPRs
        cmd[1:1] = ["-mllvm", f"-amdgpu-kernarg-preload-count={KERNARG_PRELOAD[src]}"]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-O2", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-x", "c++", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
