"""Build the gfx950 shared library ``libmoe_mi355x.so`` in-tree with hipcc.

Every source under ``csrc/`` is compiled for gfx950 only and linked into one
shared object next to this file; the Python binding loads it from there.
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
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["moe_api.cpp", "route.hip", "permute.hip", "ffn.hip", "combine.hip", "eplb.hip",
           "noalloc.hip"]

# Packed-FP32 VALU forms stay disabled in device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the ROCm toolchain is needed to build the library")
    return h


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libmoe_mi355x.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    # measurement helper: HBM stream / copy probe (bench calibration only)
    probe = os.path.join(PKG, "moe_bwprobe")
    cmd = [hipcc(), *COMMON, os.path.join(CSRC, "bwprobe.hip"), "-o", probe + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the bandwidth probe failed:\n{r.stdout}\n{r.stderr}")
    os.replace(probe + ".tmp", probe)
    if verbose:
        print(f"built {LIB_PATH} and {probe}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
