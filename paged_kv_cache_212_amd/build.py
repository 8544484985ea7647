"""Builds the HIP library ``libpa212.so`` for gfx950 in-tree with hipcc.

Usage: ``python -m paged_kv_cache_212_amd.build`` (or ``build()``).  Every
call recompiles.  Objects go to ``_build/`` at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa212.so")

ARCH = "gfx950"
SOURCES = ["pa_status.cpp", "block_manager.cpp", "pa_cache.hip", "pa_decode.hip",
           "pa_prefill.hip", "pa_prefill_pp.hip"]
# Extra compiler flags per source: the ping-pong prefill kernel takes the
# max-ilp instruction scheduler (1.3% faster on the chunked prefill; the
# other prefill kernel, in pa_prefill.hip, is slower under it).
EXTRA_FLAGS = {"pa_prefill_pp.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _flags(src: str):
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
    if src.endswith(".hip"):
        # -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
        return common + ["-x", "hip", f"--offload-arch={ARCH}", "-ffp-contract=fast",
                         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + \
            EXTRA_FLAGS.get(src, [])
    return common


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + _flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
