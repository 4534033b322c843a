"""Build libekv.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m mixed_precision_paged_amd.build [-v]
Compiles every csrc/*.hip into _build/*.o (in parallel) and links
mixed_precision_paged_amd/libekv.so.  hipcc cross-compiles for gfx950 without
a GPU present.
"""
from __future__ import annotations

import concurrent.futures
import glob
import hashlib
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libekv.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
    # packed fp32 VALU ops stay off (device feature; the host pass ignores it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def source_files():
    """The files libekv.so is built from: csrc/*.hip, csrc/*.hpp and include/ekv.h."""
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")))
    return files + [os.path.join(ROOT, "include", "ekv.h")]


def source_hash() -> str:
    """sha256 over the sources' names and code (comments and whitespace removed, so an edit
    of a comment does not change it); baked into the library as ekv_build_id()."""
    h = hashlib.sha256()
    for f in source_files():
        with open(f, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(os.path.relpath(f, ROOT).encode() + b"\0" + " ".join(text.split()).encode() + b"\0")
    return h.hexdigest()


def check_library_matches_sources() -> None:
    """Raise if the loaded libekv.so was not built from the sources in this tree."""
    from . import ekv

    built, here = ekv.ekv_build_id(), source_hash()
    if built != here:
        raise RuntimeError(f"libekv.so was built from other sources (build id {built[:16]}, tree {here[:16]}): "
                           "rebuild with `python -m mixed_precision_paged_amd.build`")


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libekv)")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    jobs = []
    build_id = f"-DEKV_BUILD_ID=\"{source_hash()}\""
    for src in sources:
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        jobs.append([hipcc, *COMMON, build_id, "-c", src, "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
