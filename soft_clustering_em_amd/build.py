"""Build libgmm.so (the HIP library behind include/gmm.h) for gfx950 with hipcc.

Each translation unit is compiled in parallel, then linked into
soft_clustering_em_amd/libgmm.so, next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgmm.so")
SOURCES = ["gmm_api.hip", "gmm_aux.hip", "gmm_estep.hip", "gmm_topm.hip", "gmm_largek.hip", "gmm_ivf.hip", "gmm_kmeans.hip", "gmm_fisher.hip", "gmm_topk.hip", "gmm_kde.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         # packed fp32 VALU ops stay disabled for every kernel in this library
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# per-file additions: the E-step kernels never form a NaN (dead components
# carry -inf or a finite floor, and every exponent of a difference is guarded),
# so min/max need no NaN quieting and fold with their DPP operands
_NONAN = ["-fno-honor-nans", "-mno-amdgpu-ieee"]
EXTRA = {"gmm_largek.hip": _NONAN, "gmm_estep.hip": _NONAN}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
