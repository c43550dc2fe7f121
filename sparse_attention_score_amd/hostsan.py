"""A host-sanitized build of the library for CPU checks of the C boundary.

The argument checks, plan sizing and launch planning in csrc/api.cpp run on the host before
any HIP call, so they can be exercised without a GPU. This module builds a copy of the
library whose host code (api.cpp) carries AddressSanitizer and UndefinedBehaviorSanitizer
instrumentation (the kernels' objects are the ordinary ones; no device code is
instrumented), links it against the shared sanitizer runtime, and builds the plain C caller
tests/c/abi_host_check.c against it with the same runtime.

Usage: build(out_dir) -> dict of paths {"lib", "c_check", "runtime"}.
"""
from __future__ import annotations

import glob
import os
import subprocess

from . import build as _b

CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def runtime_dir() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's shared AddressSanitizer runtime is not installed")
    return os.path.dirname(hits[-1])


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed:\n{r.stdout}\n{r.stderr}")


def build(out_dir: str) -> dict:
    os.makedirs(out_dir, exist_ok=True)
    kernels = [s for s in _b.SOURCES if s.endswith(".hip")]
    objs = [os.path.join(_b.OUT_DIR, s + ".o") for s in kernels]
    if not all(os.path.exists(o) for o in objs):
        _b.build()
    api_obj = os.path.join(out_dir, "api_hostsan.o")
    # host-only instrumentation: each sanitizer flag applies to the host compilation only
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    cflags = [f for f in _b.CFLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([_b._hipcc(), *cflags, *host_san, "-I", os.path.join(_b.PKG, "..", "include"), "-c",
          os.path.join(_b.SRC, "api.cpp"), "-o", api_obj])
    rt = runtime_dir()
    lib = os.path.join(out_dir, "libsparse_attn.so")
    # a host link of the objects (no device compilation here)
    _run([CLANGXX, "-shared", "-fsanitize=address,undefined", "-shared-libsan", *objs, api_obj,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", f"-Wl,-rpath,{rt}", "-o", lib])
    exe = os.path.join(out_dir, "abi_host_check")
    root = os.path.dirname(_b.PKG)
    _run([CLANG, "-std=c11", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined", "-shared-libsan",
          "-fno-sanitize-recover=undefined", os.path.join(root, "tests", "c", "abi_host_check.c"),
          "-I", os.path.join(root, "include"), "-L", out_dir, "-lsparse_attn", f"-Wl,-rpath,{out_dir}",
          f"-Wl,-rpath,{rt}", "-lm", "-o", exe])
    return {"lib": lib, "c_check": exe, "runtime": os.path.join(rt, "libclang_rt.asan-x86_64.so")}
