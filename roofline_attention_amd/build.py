"""Builds libroofattn.so in-tree from the HIP sources with hipcc for gfx950.

Usage: python -m roofline_attention_amd.build   (or call build()).
Objects go to roofline_attention_amd/_build/, the library to roofline_attention_amd/libroofattn.so,
and the compiler's per-kernel resource report (registers, scratch, occupancy) to
roofline_attention_amd/libroofattn.resources.json.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
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


# The compiler's per-kernel resource report (registers, scratch, occupancy, LDS), one remark line
# per field after a "Function Name" line.
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)")
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
           "Occupancy [waves/SIMD]": "waves_per_simd", "SGPRs Spill": "sgpr_spills", "VGPRs Spill": "vgpr_spills",
           "LDS Size [bytes/block]": "static_lds_bytes"}


def parse_resources(remarks: str) -> dict:
    """Kernel name -> resource figures, from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(remarks):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[_FIELDS[key]] = int(val)
    return out


def _compile(src: str, extra=(), objdir=OBJ) -> str:
    """Compiles one source to an object; its kernels' resource report goes beside it (.res.json)."""
    out = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPFLAGS, RESOURCE_REMARKS, *extra, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    with open(out + ".res.json", "w") as f:
        json.dump(parse_resources(r.stderr), f, indent=1, sort_keys=True)
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
    resources = {}
    for o in objs:
        with open(o + ".res.json") as f:
            resources.update(json.load(f))
    with open(resources_path(lib_path), "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    if verbose:
        print(f"built {lib_path} ({len(resources)} kernels)")
    return lib_path


def resources_path(lib_path: str = LIB) -> str:
    """Where build() records the library's per-kernel resource report (JSON)."""
    return os.path.splitext(lib_path)[0] + ".resources.json"


if __name__ == "__main__":
    build(verbose=True)
    build_ceilings(verbose=True)
    sys.exit(0)
