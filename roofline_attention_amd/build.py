"""Builds libroofattn.so in-tree from the HIP sources with hipcc for gfx950.

Usage: python -m roofline_attention_amd.build   (or call build()).
Objects go to roofline_attention_amd/_build/, the library to roofline_attention_amd/libroofattn.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libroofattn.so")
SOURCES = ["attn_api.hip", "fwd_bf16.hip", "fwd_fp8.hip", "fwd_f32.hip", "decode.hip", "bwd.hip", "fused.hip"]
ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for every HIP translation unit.
HIPFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: ROCm is required to build libroofattn.so")


def _compile(src: str, extra=(), objdir=OBJ) -> str:
    out = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


CEILINGS_SRC = "ceilings.hip"
CEILINGS_EXE = os.path.join(PKG, "ceilings")


def build_ceilings(verbose: bool = False) -> str:
    """Compiles the ceiling microbenchmarks (csrc/ceilings.hip) into the `ceilings` executable."""
    tmp = CEILINGS_EXE + ".tmp"
    cmd = [hipcc(), *HIPFLAGS, os.path.join(CSRC, CEILINGS_SRC), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {CEILINGS_SRC}:\n{r.stderr}")
    os.replace(tmp, CEILINGS_EXE)
    if verbose:
        print(f"built {CEILINGS_EXE}")
    return CEILINGS_EXE


def build(verbose: bool = False, extra_flags=(), lib_path: str = LIB) -> str:
    """Compiles every source and links the library; extra_flags/lib_path build a tuning variant."""
    objdir = OBJ if lib_path == LIB else lib_path + ".objs"
    os.makedirs(objdir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda src: _compile(src, tuple(extra_flags), objdir), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
    build_ceilings(verbose=True)
    sys.exit(0)
