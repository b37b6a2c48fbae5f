"""Build libcq.so (HIP kernels + C ABI) for gfx950 with hipcc, in place.

Usage: ``python -m rotated_codebook_bit_amd.build`` or ``build()`` from
Python.  Always recompiles.  Objects go to ``rotated_codebook_bit_amd/_build``
and the library to ``rotated_codebook_bit_amd/libcq.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libcq.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["libcq_host.cpp", "quantize.hip", "dequantize.hip", "matvec.hip", "matvec_rot.hip", "upload.hip", "gemm.hip", "repack.hip", "groups.hip", "noalloc.hip"]

ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", f"-I{os.path.join(ROOT, 'include')}"]
# Device code: no packed-FP32 instructions (hipcc's host pass warns that it
# does not know this feature; the warning is harmless).
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-file flags.  matvec_rot.hip: without SLP vectorization, so that the
# binary16 norms of its load rings are not packed two to a register (the
# packing waits for the loads as soon as they are issued).
EXTRA = {"matvec_rot.hip": ["-fno-slp-vectorize"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [_hipcc(), f"--offload-arch={ARCH}", *COMMON, *EXTRA.get(src, [])]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    else:
        cmd += ["-x", "hip", "--cuda-host-only"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
