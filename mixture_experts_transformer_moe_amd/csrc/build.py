"""Build libmoe_mi355x.so from the HIP sources in this folder (hipcc, gfx950).

Objects go to <repo>/_build/; the shared library lands in the package folder,
where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
SOURCES = ["moe_api.hip", "gate.hip", "dispatch.hip", "gemm.hip", "decode_ffn.hip", "combine.hip", "expert_store.hip",
           "noalloc.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # no packed fp32 instructions from the compiler (v_pk_* fp32 forms)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # the first 16 dwords of every kernel's arguments arrive in SGPRs (no
          # dependent scalar load at the start of each launch)
          "-mllvm", "-amdgpu-kernarg-preload-count=16",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", HERE]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 6)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
