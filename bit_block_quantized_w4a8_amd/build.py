"""Compile the HIP sources of the W4A8 library into libw4a8.so (gfx950 only).

Usage: python -m bit_block_quantized_w4a8_amd.build
The shared library lands next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libw4a8.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # packed fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the fp32 epilogue reads every element,
    # and results left in AGPRs would cost one extra copy instruction each
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the W4A8 library needs ROCm's hipcc")
    return path


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", "-I", os.path.join(ROOT, "include"), "-o", obj, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)} with exit code {res.returncode}")


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libw4a8.so."""
    from concurrent.futures import ThreadPoolExecutor

    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in sources]
    workers = max(1, min(len(sources), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        list(pool.map(lambda so: _compile(so[0], so[1], verbose), zip(sources, objs)))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
