"""Builds libsparse_mqa.so (HIP kernels for gfx950 + the C ABI) in-tree.

Usage: python -m top_sparse_mqa_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
REPO_DIR = PKG_DIR.parent
CSRC = PKG_DIR / "csrc"
LIB_PATH = PKG_DIR / "libsparse_mqa.so"
SOURCES = ["fwd.hip", "bwd.hip", "abi.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the accumulator-register form made the register allocator
    # shuttle operands and accumulators between the two register files inside the hot loops
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: set HIPCC or install ROCm")


def build(verbose: bool = False) -> Path:
    """Compile every source and link the shared library; always rebuilds."""
    objdir = REPO_DIR / "_build"
    objdir.mkdir(exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = objdir / (src + ".o")
        cmd = [cc, *HIPCC_FLAGS, "-I", str(REPO_DIR / "include"), "-c", str(CSRC / src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.DEVNULL)
        objs.append(str(obj))
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
