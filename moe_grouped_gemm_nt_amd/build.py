"""Builds the gfx950 HIP library (libdg.so) in-tree with hipcc.

Usage: python -m moe_grouped_gemm_nt_amd.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libdg.so")
CEILINGS_PATH = os.path.join(PKG_DIR, "libdg_ceilings.so")
# source -> extra flags.  The fp32-promotion kernels want MFMA results in
# VGPRs, where the promotion FMAs read them; the power-of-two-scale kernels
# keep their accumulators in AGPRs.
SOURCES = {
    "fp8_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "fp8_gemm_e8m0.hip": [],
    "dg_api.hip": [],
}

# packed fp32 VALU forms are disabled on purpose: the kernels issue one fp32
# operation per VALU instruction, the form their results are tested in
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain (ROCm) is required to build libdg.so")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # the host pass does not know the packed-fp32 feature flag; that warning is expected
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


def build(verbose: bool = False, extra_flags=None) -> str:
    objdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src, flags in SOURCES.items():
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append(([hipcc()] + HIPCC_FLAGS + flags + list(extra_flags or []) +
                     ["-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    # the sources compile independently; one process each
    with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    objs = [obj for _, obj in jobs]
    tmp = LIB_PATH + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB_PATH)
    build_ceilings(verbose)
    return LIB_PATH


def build_ceilings(verbose: bool = False) -> str:
    """libdg_ceilings.so: the MFMA / memory / launch microbenchmarks (include/dg_ceilings.h)."""
    tmp = CEILINGS_PATH + ".tmp"
    _run([hipcc()] + HIPCC_FLAGS + ["-shared", "-I", INCLUDE, os.path.join(CSRC, "ceilings.hip"), "-o", tmp],
         verbose)
    os.replace(tmp, CEILINGS_PATH)
    return CEILINGS_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
