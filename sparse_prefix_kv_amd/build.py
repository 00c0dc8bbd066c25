"""Build libsprint.so in-tree with hipcc for gfx950.

Each .hip source compiles to an object in ``_build/`` (in parallel), then one
shared library is linked next to this file.  Usage: ``python -m
sparse_prefix_kv_amd.build`` or ``build()`` from Python.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsprint.so")
C_CHECK = os.path.join(ROOT, "tests", "c_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = os.environ.get("SPRINT_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

SOURCES = ["abi.hip", "score.hip", "prune.hip", "attend.hip", "lmhead.hip", "unmask.hip",
           "append.hip", "moe.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature; drop that noise
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_c_check(verbose)
    return LIB


def build_c_check(verbose: bool = True) -> str:
    """Link tests/c_abi_check.cpp, a host program that calls the library
    through include/sprint.h alone, against libsprint.so (no Python, no torch)."""
    src = os.path.join(ROOT, "tests", "c_abi_check.cpp")
    cmd = [shutil.which("g++") or "g++", "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), src,
           "-o", C_CHECK, "-L", PKG, "-lsprint", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../sparse_prefix_kv_amd", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"c_abi_check build failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {C_CHECK}")
    return C_CHECK


if __name__ == "__main__":
    build()
