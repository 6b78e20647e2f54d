"""Build libw4.so (the C-ABI library of include/w4.h) for gfx950 with hipcc.

    python w4_block_dequant_amd/build.py

(run as a script: importing the package would load the library being rebuilt)

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled and kernel-argument preloading on, then linked into
w4_block_dequant_amd/libw4.so (in-tree).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel-argument preloading: the first 14 dwords of every kernel's
    # arguments arrive in SGPRs at wave launch instead of through a scalar
    # load (the short decode launches save one memory round trip each)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    # MFMA results in ordinary VGPRs (gfx950 allows it): no accumulation-
    # register copies before the fp32 epilogue arithmetic, fewer registers
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    """Compile every source and link libw4.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
