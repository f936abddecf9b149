"""Build libsnm.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Every source is compiled to its own object (in parallel, under _build/), then the objects
are linked into structured_sparse_matrix_amd/libsnm.so.

Usage: python -m structured_sparse_matrix_amd.build   (or __graft_entry__.build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsnm.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["encode.hip", "spmm.hip", "spmm_skinny.hip", "spmm_splitk.hip", "spmm_wide.hip",
           "spmm_vnm_big.hip", "spmm_vnm_big64.hip", "attention.hip", "attention_f32.hip", "bitmap.hip", "ceilings.hip",
           "validate.cpp", "variant.cpp", "abi.cpp"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # gfx950 packed-fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# matrix-core accumulators in ordinary VGPRs: epilogues read them without v_accvgpr_read
# copies. Sources listed in AGPR_SOURCES keep the compiler's default instead: their kernels
# hold more accumulators than the ordinary VGPR file has room for.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_SOURCES: set = set()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsnm)")


def _flags(src: str):
    return COMMON_FLAGS + ([] if src in AGPR_SOURCES else VGPR_FORM)


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [hipcc(), *_flags(src), "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed on {src} with status {proc.returncode}")
    return obj


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source into structured_sparse_matrix_amd/libsnm.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"link failed with status {proc.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
