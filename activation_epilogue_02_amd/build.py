"""Build the gfx950 shared library libgemm_epilog.so in-tree with hipcc.

Each translation unit is compiled to an object in parallel, then linked.
The library links the HIP runtime by name; loaded after ``import torch`` it
binds to the runtime torch already loaded, so streams and device pointers
from torch are valid in it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgemm_epilog.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "tile_launch.hip", "tile_f32.hip", "tile_f16.hip", "tile_bf16.hip", "tile_f8.hip",
           "tile2_f16_f16.hip", "tile2_f16_f32.hip", "tile2_bf16_bf16.hip", "tile2_bf16_f32.hip",
           "tile2_f8_bf16.hip", "tile2_f8_f16.hip", "tile2_f8_f32.hip",
           "tile2_mx_bf16.hip", "tile2_mx_f16.hip", "tile2_mx_f32.hip",
           "tile2_bf16_f8.hip", "tile2_f16_f8.hip", "tile2_f8_f8.hip", "tile2_mx_f8.hip",
           "smallm_kernel.hip", "ew_kernel.hip"]

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Wall", "-Wno-unused-result",
          # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # let `#pragma unroll` unroll the tile epilogue fully: past the
          # default size limit the loop stays rolled, its accumulator index
          # becomes dynamic and the accumulators move to scratch memory
          "-mllvm", "-pragma-unroll-threshold=1000000"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libgemm_epilog.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
