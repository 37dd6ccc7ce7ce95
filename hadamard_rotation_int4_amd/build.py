"""Build libhr.so in-tree with hipcc for gfx950.

Usage: python hadamard_rotation_int4_amd/build.py   (or call build()).  Run it as
a script (or load it by path): importing the package first would try to load
the very library this builds.
Each .hip file under csrc/ is compiled to an object in parallel, then linked
into hadamard_rotation_int4_amd/libhr.so.  The hash of the sources
(srchash.py) is compiled in as hr_build_id(), which the binding checks.
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
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libhr.so")

ARCH = "gfx950"
# Packed-fp32 VALU forms are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _source_hash() -> str:
    # srchash.py sits beside this file; load it by path (the package itself
    # would try to load the library being built)
    import importlib.util
    spec = importlib.util.spec_from_file_location("hr_srchash", os.path.join(PKG, "srchash.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.source_hash()


def _compile(src: str, defines=()) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, *defines, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (r.stderr or "").splitlines() if ln.strip() and noise not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    defines = [f'-DHR_SOURCE_HASH="{_source_hash()}"']
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, defines), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
