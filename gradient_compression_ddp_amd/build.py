"""Build libgc.so (the HIP kernels for gfx950 and the C ABI) in-tree with hipcc.

Flags: -O3, -ffp-contract=off (no fused multiply-add, so every float operation rounds
once, as the numeric contract requires), IEEE division and square root (hipcc's default),
denormals kept (the default on gfx950), and packed-fp32 instruction selection turned off.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgc.so")
ARCH = "gfx950"

SOURCES = ["capi.cpp", "minmax.hip", "qsgd.hip", "terngrad.hip", "ef_topk.hip",
           "powersgd.hip", "decompress.hip", "noalloc.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libgc.so")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    hip = src.endswith(".hip")
    # the language flag must come before the source it applies to
    cmd = [hipcc()] + (["-x", "hip"] if hip else []) + ["-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS
    if hip:
        cmd += HIP_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    if res.stderr.strip() and verbose:
        print(res.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 7) -> str:
    """Compile every source for gfx950 and link libgc.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libgc.so failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
