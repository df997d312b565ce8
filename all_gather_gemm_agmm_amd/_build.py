"""Build libagmm.so (HIP, gfx950) in-tree.

    python -m all_gather_gemm_agmm_amd._build

Every source is compiled by hipcc for gfx950 only.  Packed-fp32 VALU forms are
disabled for all device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libagmm.so")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Per-source extra flags.  The MFMA GEMM asks the machine scheduler to favour
# latency hiding (it keeps several LDS fragment loads in flight ahead of the
# MFMAs instead of minimising register pressure).
SOURCES = {
    "agmm_api.cpp": [],
    "gather_f32.hip": [],
    "gemm_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "skinny.hip": [],
    "noalloc.hip": [],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libagmm.so)")


def _compile(src: str, extra, out_dir: str, verbose: bool) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libagmm.so next to this file."""
    with tempfile.TemporaryDirectory(prefix="agmm_build_") as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            futs = [ex.submit(_compile, s, f, tmp, verbose) for s, f in SOURCES.items()]
            objs = [f.result() for f in futs]
        out_tmp = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
