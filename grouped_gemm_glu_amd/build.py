"""Build libmoeglu.so (the HIP library) in-tree for gfx950 with hipcc.

Usage:  python grouped_gemm_glu_amd/build.py [--jobs N] [--verbose]

Each .hip translation unit is compiled to an object in parallel, then linked
into grouped_gemm_glu_amd/libmoeglu.so.  Every HIP compile disables the
packed-fp32 instruction forms (-packed-fp32-ops).  The build always runs (no
up-to-date check) so that a changed source can never be shadowed by a stale
library.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libmoeglu.so")
# (source, object name, extra flags): the activation kernels are compiled once
# per activation (MOE_ACT = the moe_act_t value), which also spreads the
# largest translation units over more parallel jobs.
SOURCES = ([("api.hip", "api", []), ("gemm_fwd.hip", "gemm_fwd", []), ("gemm_bwd.hip", "gemm_bwd", []),
            ("gemm_mx.hip", "gemm_mx", []), ("gemm_wgrad.hip", "gemm_wgrad", []),
            ("gemm_wgrad_mx.hip", "gemm_wgrad_mx", [])]
           + [(f"gemm_act_{d}.hip", f"gemm_act_{d}_{a}", [f"-DMOE_ACT={a}"])
              for d in ("bwd", "fwd") for a in range(4)])
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoeglu.so)")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def compile_one(unit, verbose: bool) -> str:
    src, name, extra = unit
    obj = os.path.join(OBJDIR, name + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + common_flags() + extra
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_host_asan(jobs: int = 8, verbose: bool = False) -> str:
    """A copy of the library whose entry points (api.hip) have their HOST code
    built with AddressSanitizer; device code and the other units are compiled
    as usual (objects of an earlier build() are reused).  For the CPU-only
    argument-validation test; load it with the ASan runtime preloaded.
    Returns _build/asan/libmoeglu_asan.so."""
    asan_dir = os.path.join(ROOT, "_build", "asan")
    os.makedirs(asan_dir, exist_ok=True)
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    todo = []
    for unit in SOURCES:
        src, name, extra = unit
        if name == "api":
            continue
        obj = os.path.join(OBJDIR, name + ".o")
        objs.append(obj)
        if not os.path.exists(obj):
            todo.append(unit)
    if todo:
        with ThreadPoolExecutor(max(1, jobs)) as ex:
            list(ex.map(lambda s: compile_one(s, verbose), todo))
    api_obj = os.path.join(asan_dir, "api_asan.o")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = ([hipcc(), "-c", os.path.join(CSRC, "api.hip"), "-o", api_obj] + common_flags()
           + host_asan + ["-g"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (host ASan) failed on api.hip:\n{r.stdout}\n{r.stderr}")
    lib = os.path.join(asan_dir, "libmoeglu_asan.so")
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", lib + ".tmp", api_obj] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (host ASan) failed:\n{r.stdout}\n{r.stderr}")
    os.replace(lib + ".tmp", lib)
    return lib


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()
