"""Hash of the library's sources (every file under csrc/ and include/hr.h).

The build compiles it into libhr.so (hr_build_id()); the binding recomputes it
at import and refuses a library built from other sources.  Plain file reads
only, so it can be loaded before the library exists.
"""
from __future__ import annotations

import glob
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)


def source_files():
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "hr.h"))
    return [f for f in files if os.path.isfile(f)]


def source_hash() -> str:
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:32]
