"""Build libcfc_amd.so (gfx950) in-tree with hipcc.

Usage: python -m cfc_recurrent_cell_amd.build   (or build_library() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "cfc.hip")
LIB = os.path.join(PKG, "libcfc_amd.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    # no packed FP32 instructions: only scalar / f64 VALU forms are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # loops start on 64-byte boundaries: the serial chains' loop bodies
    # measured up to 4 % slower when an unrelated edit shifted their start
    "-falign-loops=64",
    # matrix-core results in architectural VGPRs: the weight-gradient tiles
    # are converted to float32 straight from them instead of being copied out
    # of accumulation registers first (the training-scale fused kernel then
    # issues 680 fewer copies and ran 0.7 % faster on MI355X)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


def build_library(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
