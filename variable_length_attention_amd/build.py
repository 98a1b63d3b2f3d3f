"""Builds the HIP library ``libvarlen_attn.so`` in-tree for gfx950.

Every translation unit is compiled by hipcc (``--offload-arch=gfx950``) into
``_build/`` in parallel, then linked into the package directory.  Packed
fp32 arithmetic is disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvarlen_attn.so")
# attainable-rate probes for the benchmark's roofline context (not the library)
PROBE_LIB = os.path.join(PKG, "libva_probe.so")
PROBE_SOURCES = ["va_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["va_api.cpp", "va_plan.hip", "va_prefill_bf16.hip", "va_prefill_f32.hip", "va_decode.hip",
           "va_check.hip", "va_backward.hip", "va_merge.hip", "va_sparse.hip", "va_window.hip", "va_prefill512.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-command-line-argument"]
# Per-file device options.  The backward's dK/dV kernel and the d512 sparse
# shared-KV and dense forward kernels keep their accumulators in AGPRs
# through inline assembly
# and need every other matrix instruction in the VGPR form (the backend
# otherwise picks the AGPR form for a whole kernel that may use more than
# 256 registers).
EXTRA = {"va_backward.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=1"],
         "va_sparse.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=1"],
         "va_prefill512.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, objs[len(SOURCES):])):
        tmp = lib + f".tmp{os.getpid()}"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *lib_objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
