"""Build libmlra.so in-tree for gfx950 with hipcc.

    python -m long_context_decode_mlra_amd.build        # or build() from Python

Always recompiles. The library lands next to this file, where the binding loads it.
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
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmlra.so")
BUILD_DIR = os.path.join(ROOT, "_build")

# HIP translation units of the library, compiled in parallel.
HIP_SOURCES = ("mlra_attention.hip", "mlra_combine.hip", "mlra_absorb.hip", "mlra_probes.hip",
               "gqa_attention.hip", "mlra_noalloc.hip")

ARCH = "gfx950"
# Packed-fp32 VALU forms are kept out of every kernel.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extras. The one-wave-per-branch attention kernel runs one wave per SIMD; without
# the MFMA VGPR form the compiler keeps its accumulators in AGPRs and copies them to and from
# VGPRs every tile. The bf16 kernels that fit in 256 VGPRs compile to the same code either
# way; the fp32 kernels that need more keep fewer values in AGPRs.
SOURCE_FLAGS = {"mlra_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmlra.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    params_o = os.path.join(BUILD_DIR, "mlra_params.o")
    # Host-only C++ (no HIP): validation and workspace sizing.
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-c",
          os.path.join(CSRC, "mlra_params.cpp"), "-o", params_o])
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in HIP_SOURCES]
    with ThreadPoolExecutor(max_workers=len(HIP_SOURCES)) as ex:
        outs = list(ex.map(lambda so: _run([hipcc, *HIP_FLAGS, *SOURCE_FLAGS.get(so[0], []), "-Wall", "-I",
                                            INCLUDE, "-c", os.path.join(CSRC, so[0]), "-o", so[1]]),
                           zip(HIP_SOURCES, objs)))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", params_o, *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
