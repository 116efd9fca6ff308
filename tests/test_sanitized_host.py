"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, without a
GPU: the CPU oracle (compiled with clang, -fsanitize=address,undefined) and
the library's host side -- the C-ABI validators, workspace sizing and
launch planning -- compiled with the sanitizers on the host pass only (GPU
code is built as usual). The oracle pins, the C-ABI rejection tests and the
binding tests then run in a fresh interpreter against those two builds,
with the sanitizer runtime preloaded; any finding aborts that run."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def _asan_runtime():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    base = os.path.dirname(os.path.dirname(os.path.realpath(CLANG)))
    for root, _, files in os.walk(os.path.join(base, "lib")):
        if "libclang_rt.asan-x86_64.so" in files:
            return os.path.join(root, "libclang_rt.asan-x86_64.so")
    return None


def _build_lib_module():
    spec = importlib.util.spec_from_file_location(
        "_tsd_build_lib_san", os.path.join(ROOT, "top_sparse_decode_amd",
                                           "build_lib.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_host_code_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if not os.path.exists(CLANG) or rt is None:
        pytest.skip("clang sanitizer runtime not installed")
    oracle_so = str(tmp_path / "libtsd_oracle_san.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared",
                    "-shared-libasan", *SAN,
                    os.path.join(ROOT, "oracle", "tsd_oracle.c"), "-o",
                    oracle_so, "-lm"], check=True)
    host = []
    for f in SAN:
        host += ["-Xarch_host", f]
    lib_so = _build_lib_module().build(
        out=str(tmp_path / "libtsd_san.so"), build_dir=str(tmp_path / "obj"),
        host_flags=host + ["-shared-libasan"])
    env = dict(os.environ, LD_PRELOAD=rt, TSD_LIB=lib_so,
               TSD_ORACLE_LIB=oracle_so,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_pins.py", "test_abi.py", "test_binding.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p",
                        "no:cacheprovider", "-m", "not gpu", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "error" not in r.stdout.lower(), tail
