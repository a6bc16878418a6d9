"""Build libglance.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m tree_verified_block_amd.build

Each source compiles to an object under tree_verified_block_amd/_build/ (in
parallel), then hipcc links them into tree_verified_block_amd/libglance.so.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libglance.so")
SOURCES = ["glance.cpp", "tree.hip", "gemm.hip", "attn.hip", "walk.hip", "layer.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags(src: str):
    f = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", f"-I{INCLUDE}", f"-I{CSRC}",
         "-Wall", "-Wno-unused-function"]
    if src.endswith(".hip"):
        # keep the compiler from emitting packed fp32 arithmetic in device code
        f += ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    return f


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *_flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
