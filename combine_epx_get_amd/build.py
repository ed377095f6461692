"""Build libepx.so (HIP for gfx950) in-tree, and its bounds-checked twin.

Usage: python -m combine_epx_get_amd.build  (or __graft_entry__.build()).

Each .hip source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into combine_epx_get_amd/libepx.so. The same sources
compiled with EPX_CHECKED (objects in _build/checked/) give
libepx_checked.so, in which every computed row index is checked before its
access (a debugging aid; the binding loads it when EPX_LIBRARY names it).
Device code is built for gfx950 only, with packed-fp32 instructions
disabled and no floating-point contraction (the kernels state every fma
they want).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libepx.so")
LIB_CHECKED = os.path.join(PKG, "libepx_checked.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, checked: bool) -> str:
    out_dir = os.path.join(BUILD, "checked") if checked else BUILD
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DEPX_CHECKED"] if checked else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, "checked"), exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = [(src, checked) for checked in (False, True) for src in sources]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(sources)
    _link(objs[:n], LIB)
    _link(objs[n:], LIB_CHECKED)
    if verbose:
        print(f"built {LIB} and {LIB_CHECKED}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
