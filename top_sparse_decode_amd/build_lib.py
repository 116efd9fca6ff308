"""Builds libtsd.so in-tree with hipcc for gfx950.

    python top_sparse_decode_amd/build_lib.py

(Run it as a script: importing the package itself loads the built library.)
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import importlib.util
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


# Every HIP source is compiled with packed-FP32 code generation disabled,
# and with kernel-argument preloading: gfx950 loads the first kernel
# arguments (up to 16 dwords, 14 here beside the argument-buffer pointer)
# into scalar registers at wave launch, so a kernel's first memory loads
# need not wait for a scalar load of the argument buffer (the kernels put
# the arguments those loads need first). The code object keeps a prologue
# that loads them itself where the firmware does not preload.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                "-Wall", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-mllvm", "-amdgpu-kernarg-preload-count=16",
                "-I" + INCLUDE, "-I" + CSRC]


# Per-source extra flags. The index scans assume NaN-free scores (a NaN
# score is outside the top-k contract), which lets max(0, x) compile to one
# v_max_f32 instead of a NaN-quieting max followed by the max.
EXTRA_FLAGS = {"score_qsa.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) +
                  glob.glob(os.path.join(CSRC, "*.cpp")))


def _source_sha256() -> str:
    spec = importlib.util.spec_from_file_location(
        "_tsd_srchash", os.path.join(PKG, "_srchash.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.source_sha256()


def _compile(src: str, digest: str, build_dir: str = None,
             extra: list = ()) -> str:
    build_dir = build_dir or BUILD
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = ([hipcc()] + DEVICE_FLAGS + EXTRA_FLAGS.get(os.path.basename(src), [])
           + [f'-DTSD_SOURCE_SHA256="{digest}"'] + list(extra)
           + ["-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, build_dir: str = BUILD,
          host_flags: list = ()) -> str:
    """Compile every source and link libtsd.so (always rebuilds).
    ``host_flags`` are added to every compile and to the link (a sanitized
    variant passes host-only sanitizer flags here, with ``out`` and
    ``build_dir`` elsewhere)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    digest = _source_sha256()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, digest, build_dir,
                                              host_flags), srcs))
    tmp = out + ".tmp"
    cmd = ([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"]
           + list(host_flags) + objs + ["-o", tmp])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def ensure_built() -> str:
    """Build only when no library exists yet."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
