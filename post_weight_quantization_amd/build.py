"""Build libgptq_mi355x.so in-tree with hipcc for gfx950 (every call recompiles)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgptq_mi355x.so")
SOURCES = ["fold.hip", "fold64.hip", "sweep.hip", "gram.hip", "debias.hip", "act_order.hip", "api.hip",
           "check.hip", "round.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-ffp-contract=fast-honor-pragmas", "-fno-gpu-rdc",
         # The sweep's column loops are sized for the unroller before their lane broadcasts fold
         # to single DPP moves; left rolled, each broadcast becomes a branch tree.
         "-mllvm", "-pragma-unroll-threshold=200000"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # Every unroll pragma must take effect (a build error rather than a slow kernel).
    if "loop not unrolled" in r.stderr:
        raise RuntimeError(f"hipcc left a loop rolled in {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "-shared", f"--offload-arch={ARCH}", "-fPIC", "-pthread", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
