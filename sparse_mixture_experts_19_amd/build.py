"""Build ``libmoe_mi355x.so`` in-tree for gfx950 with hipcc.

Usage: ``python -m sparse_mixture_experts_19_amd.build`` (or call ``build()``).
Each HIP source compiles to an object under ``_build/`` (in parallel), then
one shared library is linked next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "route.hip", "permute.hip", "round.hip", "gemm_mfma.hip", "gemm_f32.hip", "mxfp8.hip", "backward.hip",
           "combine.hip"]

# Per-source flags.  route.hip: its MFMA results are added on the vector ALU
# right away, so they are kept in VGPRs (no copies out of AGPRs per MFMA).
SOURCE_FLAGS = {"route.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 instructions are left to nobody: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{SRC}",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{p.stdout}")
    return p.stdout


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    _run([HIPCC, *CFLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(SRC, src), "-o", obj])
    return obj


def build(verbose: bool = False, jobs: int = 8, extra=()) -> str:
    """Compile every HIP source for gfx950 and link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra=tuple(sys.argv[1:]))
