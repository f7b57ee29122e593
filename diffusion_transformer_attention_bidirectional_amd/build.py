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
# The host units are plain C++ (hipcc would otherwise compile a .cpp file as HIP source
# for a default GPU as well).
HOST = ["-x", "c++", "-I", "/opt/rocm/include"]
# -fno-honor-nans: from finite inputs no kernel produces or consumes a NaN: masked scores
# are -inf and never meet another -inf (the running max starts finite), and the max-skip
# rule keeps every probability finite in the P operand's type (at most 2^24 in bf16, 2^15
# in fp16), so max reductions need no NaN-quieting instructions.
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
        ("plan.cpp", COMMON + HOST),
        ("capi.cpp", COMMON + HOST + ["-D__HIP_PLATFORM_AMD__"]),
        ("gemm.cpp", COMMON + HOST + ["-D__HIP_PLATFORM_AMD__"]),
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


SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libkrea_attn_san.so")
# Host-only checking build: the planner, the C ABI and the GEMM glue built by the host
# compiler with AddressSanitizer and UndefinedBehaviorSanitizer; the kernels unit is built
# as usual (no GPU code is instrumented).  Load it with KREA_ATTN_LIB=<path> and the
# sanitizer runtime preloaded (see sanitize_env()).
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined", "-g", "-O1"]


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    gxx = shutil.which("g++") or "g++"
    objs = []
    for src in ("plan.cpp", "capi.cpp", "gemm.cpp"):
        obj = os.path.join(SAN_DIR, src + ".o")
        _run([gxx, "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC, "-I", "/opt/rocm/include",
              "-D__HIP_PLATFORM_AMD__"] + SAN_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    kobj = os.path.join(SAN_DIR, "kernels.hip.o")
    _run([hipcc()] + COMMON + DEVICE + ["-c", os.path.join(CSRC, "kernels.hip"), "-o", kobj])
    _run([gxx, "-shared", "-o", SAN_LIB] + objs + [kobj] + SAN_FLAGS[:1] +
         ["-L/opt/rocm/lib", "-lamdhip64", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"])
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


def sanitize_env() -> dict:
    """Environment that runs Python with the sanitized library: the sanitizer runtimes
    preloaded (Python itself is not instrumented), leak checks off (the interpreter's own
    allocations at exit are not the library's)."""
    gxx = shutil.which("g++") or "g++"
    libs = [subprocess.run([gxx, f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
            for n in ("libasan.so", "libubsan.so")]
    env = dict(os.environ)
    env.update(LD_PRELOAD=":".join(libs), KREA_ATTN_LIB=SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--sanitize":
        build_sanitized(verbose=True)
        # the host ABI tests against the sanitized library
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", os.path.join(ROOT, "tests", "test_host_abi.py")],
                           env=sanitize_env(), cwd=ROOT)
        sys.exit(r.returncode)
    build(verbose=True)
    sys.exit(0)
