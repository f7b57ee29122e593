"""Build libkrea_attn.so for gfx950 (MI355X) in this package directory.

Four translation units: the host planner (plan.cpp), the C ABI (capi.cpp) and the block
path's GEMM calls (gemm.cpp, linked against hipBLASLt) as host C++, the kernels
(kernels.hip) as HIP for gfx950.  Flags:
  -Xclang -target-feature -Xclang -packed-fp32-ops  no packed fp32 VALU instructions
  -mllvm -amdgpu-mfma-vgpr-form                      keep MFMA results in VGPRs (the
      softmax reads the score accumulators directly; AGPR results would need a
      v_accvgpr_read per element)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkrea_attn.so")
BUILD = os.path.join(PKG, "_build")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall"]
# -fno-honor-nans: no kernel produces or consumes a NaN (masked scores are -inf and the
# running max starts finite), so max reductions need no NaN-quieting instructions.
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    units = [
        ("plan.cpp", COMMON),
        ("capi.cpp", COMMON + ["-D__HIP_PLATFORM_AMD__"]),
        ("gemm.cpp", COMMON + ["-D__HIP_PLATFORM_AMD__"]),
        ("kernels.hip", COMMON + DEVICE),
    ]
    jobs = []
    for src, flags in units:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(([cc] + flags + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(lambda j: _run(j[0]), jobs))
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs] +
         ["-L/opt/rocm/lib", "-lhipblaslt"])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
