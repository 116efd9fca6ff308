"""SHA-256 of the sources libtsd.so is built from.

The build compiles the digest into the library (``tsd_source_sha256``), and
the binding recomputes it from the sources beside the library at import, so
a library built from other sources (a stale binary copied along with a
changed tree) is refused instead of silently run. The digest covers every
file under ``csrc/``, the public header and the build script (its compiler
flags change the code), each as its relative path and bytes.
"""
from __future__ import annotations

import glob
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)


def source_files(pkg=PKG, root=ROOT):
    csrc = os.path.join(pkg, "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*")))
    files = [f for f in files if os.path.isfile(f)]
    return files + [os.path.join(root, "include", "tsd.h"),
                    os.path.join(pkg, "build_lib.py")]


def source_sha256(pkg=PKG, root=ROOT):
    """Hex digest, or None when a source file is missing."""
    h = hashlib.sha256()
    for f in source_files(pkg, root):
        if not os.path.exists(f):
            return None
        rel = os.path.relpath(f, root).replace(os.sep, "/")
        h.update(rel.encode() + b"\0")
        with open(f, "rb") as fh:
            data = fh.read()
        h.update(len(data).to_bytes(8, "little") + data)
    return h.hexdigest()
