"""Builds libcpattn.so (the HIP library behind include/cp_attn.h) in-tree for gfx950."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcpattn.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off: the compiler emits plain fp32 ops instead
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-file extra flags. The bf16 attention kernel never produces NaN, so its
# fmax reductions need no NaN canonicalisation (v_max3_f32 directly).
FILE_FLAGS = {"attn_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return h


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o",
           obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libcpattn.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    build_c_abi_check(verbose)


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi", "abi_check")


def build_c_abi_check(verbose: bool = False) -> None:
    """Compile the plain-C99 program that drives the ABI through include/cp_attn.h
    (gcc, HIP runtime C API, linked against the library just built)."""
    if not os.path.exists(C_CHECK_SRC):
        return
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), C_CHECK_SRC,
           "-o", C_CHECK_BIN, "-L", PKG, "-lcpattn", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/../../context_attention_dit_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {C_CHECK_SRC}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {C_CHECK_BIN}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
