"""A host program that drives libepx through the C ABI alone (no Python in
its process), and its build: the GPU test tests/test_c_abi_gpu.py runs it
and compares what it wrote with the oracle."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "epx_abi_driver.cpp")
EXE = os.path.join(HERE, "epx_abi_driver")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    """Compile the driver against include/epx.h and link it to the in-tree
    libepx.so (found at run time through a path relative to the program)."""
    lib_dir = os.path.join(ROOT, "combine_epx_get_amd")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall", "-Wextra",
           "-I", os.path.join(ROOT, "include"), SRC, "-L", lib_dir, "-l:libepx.so",
           "-Wl,-rpath,$ORIGIN/../../combine_epx_get_amd", "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the ABI driver failed:\n{r.stdout}\n{r.stderr}")
    return EXE
