"""Build libsparse_attn.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python sparse_attention_score_amd/build.py [--jobs N]   (runs without importing the package)
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsparse_attn.so")
SOURCES = ["indexer.hip", "select.hip", "attn.hip", "compress.hip", "api.cpp"]
HEADERS = ["sa_device.h", "sa_launch.h"]
ARCH = os.environ.get("SPARSE_ATTN_ARCH", "gfx950")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep hand-written float code on scalar VALU ops (no packed fp32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no kernel relies on NaN semantics (infinities are still honoured): lets fmaxf fold
    # into DPP max instructions without canonicalising its inputs
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the library needs ROCm to build")
    return h


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, "-I", os.path.join(PKG, "..", "include"), "-c", os.path.join(SRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    """Compile every source and link the shared library; always rebuilds."""
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    sys.exit(0)
