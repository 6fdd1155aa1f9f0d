"""Build libssd.so (the SSD C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m mamba_ssd_chunked_amd.csrc.build   (or build() from Python)
The library lands next to the Python binding as mamba_ssd_chunked_amd/libssd.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libssd.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")

HIP_SOURCES = ["k_modules.hip", "k_fused.hip", "k_fused_i8.hip", "k_chunked_i8.hip", "k_calib.hip",
               "k_decode.hip", "k_epilogue.hip", "ssd_noalloc.hip"]
CPP_SOURCES = ["ssd_api.cpp"]

ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", f"-I{HERE}"]
# Packed fp32 VALU ops are kept off; the compiler's host pass warns that it
# does not know the feature, which is harmless.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libssd.so)")


def _compile(src: str, hip: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON]
    if hip:
        cmd += HIP_FLAGS
    cmd += ["-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = [(s, True) for s in HIP_SOURCES] + [(s, False) for s in CPP_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
