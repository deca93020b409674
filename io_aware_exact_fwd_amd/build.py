"""Compile the gfx950 attention library ``libattn.so`` in-tree with hipcc.

Every HIP translation unit is built for gfx950 only (no other target, no
CUDA path).  Packed-fp32 instructions are disabled in device code: the
kernels' fp32 arithmetic stays on plain VALU ops.

    python -m io_aware_exact_fwd_amd.build [--verbose]
"""
from __future__ import annotations

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
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_fwd_fp8.hip"]
HEADERS = ["attn_device.h", "attn_launch.h", "attn_layout.h"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
          "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def hipcc() -> str:
    h = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError(f"hipcc not found ({h})")
    return h


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:  # host-only C++ against the HIP runtime API
        cmd = [hipcc(), *COMMON, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link ``libattn.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libattn.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
