"""Builds libmoedecode.so in-tree with hipcc for gfx950.

    python -m bit_quantized_expert_softmax_amd.build

Every source is compiled on each call (objects under ``_build/``), then
linked into ``bit_quantized_expert_softmax_amd/libmoedecode.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoedecode.so")

# plain C++ (no HIP headers)
HOST_SOURCES = ["lfu.cpp", "store.cpp"]
# compiled as HIP: kernels, and host code that calls the HIP runtime
HIP_SOURCES = ["abi.cpp", "layer.cpp", "route.hip", "decode.hip", "gemv.hip", "prefill.hip", "batched.hip", "attn.hip", "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-command-line-argument",
          f"-I{os.path.join(ROOT, 'include')}"]
# Packed fp32 VALU ops are kept out of the generated code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
    if src in HIP_SOURCES:
        cmd = [hipcc(), "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), "-x", "c++", *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = HOST_SOURCES + HIP_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
