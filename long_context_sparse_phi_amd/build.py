"""Build the NSA HIP library (libnsa.so) for gfx950, in-tree.

Each translation unit under csrc/ is compiled by hipcc into _build/, in
parallel, and linked into long_context_sparse_phi_amd/libnsa.so.  Runs on a
machine without a GPU (hipcc cross-compiles).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libnsa.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are disabled: only plain scalar fp32 ops are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: with the AGPR form the compiler copied
    # loop-carried accumulators into AGPRs and back on every iteration
    # (hundreds of v_accvgpr moves per tile in the dK/dV, selected-branch and
    # decode loops)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]
SOURCES = ["nsa_api.cpp", "nsa_gemm.hip", "nsa_phi.hip", "nsa_cmp.hip", "nsa_attn.hip", "nsa_decode.hip", "nsa_bwd.hip",
           "nsa_append.hip"]


# Per-file additions.  The compressed-branch kernels never carry NaN through
# their softmax (masked scores are -inf, never NaN), so max/min need no NaN
# quieting there.
FILE_FLAGS = {"nsa_cmp.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
