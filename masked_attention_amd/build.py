"""Build librk.so (the HIP/CDNA4 library behind include/rk.h) with hipcc.

Usage: python -m masked_attention_amd.build  (or build() from Python).
Always recompiles.  Output: masked_attention_amd/librk.so.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "librk.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "plan.hip", "rope.hip", "attn_ref.hip", "attn_mfma.hip", "attn_combine.hip",
           "attn_bwd_ref.hip", "attn_bwd_mfma.hip", "layout.cpp", "gather_sum.hip",
           "attn_pointwise_ref.hip", "attn_pointwise_mfma.hip", "norm_bwd.hip", "scratch.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]
# Packed-fp32 VALU forms are kept out of the device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build librk)")


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src + ".o")
        # every source, the host-only .cpp files included, is compiled as HIP
        # (they use the HIP runtime's types and launch the kernels)
        cmd = [hipcc, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
