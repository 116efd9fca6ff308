"""Builds libtsd.so in-tree with hipcc for gfx950.

    python top_sparse_decode_amd/build_lib.py

(Run it as a script: importing the package itself loads the built library.)
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtsd.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Every HIP source is compiled with packed-FP32 code generation disabled.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                "-Wall", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-I" + INCLUDE, "-I" + CSRC]


# Per-source extra flags. The index scans assume NaN-free scores (a NaN
# score is outside the top-k contract), which lets max(0, x) compile to one
# v_max_f32 instead of a NaN-quieting max followed by the max.
EXTRA_FLAGS = {"score_qsa.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) +
                  glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ([hipcc()] + DEVICE_FLAGS + EXTRA_FLAGS.get(os.path.basename(src), [])
           + ["-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libtsd.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + [
        "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def ensure_built() -> str:
    """Build only when no library exists yet."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
