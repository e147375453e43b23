"""Build libsvdq.so (HIP kernels for gfx950 + host pack) in-tree.

    python -m diffusion_smooth_group_amd.build

Compiles every time it is called.  Device code: hipcc for gfx950 only, with
packed-FP32 instructions disabled and no floating-point contraction (the
quantizers must round exactly as written).  Host code: the pack and the
exports with -ffp-contract=off; the SVD (Gram matrix, Lanczos) with AVX2 and
FMA.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsvdq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-I" + os.path.join(ROCM, "include"),
              "-I" + os.path.join(ROOT, "include"), "-D__HIP_PLATFORM_AMD__", "-Wall"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cxx = shutil.which("g++") or "g++"
    objs = []
    for name in ("svdq_kernels", "svdq_probe"):
        obj = os.path.join(BUILD, name + ".o")
        _run([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, name + ".hip"), "-o", obj])
        objs.append(obj)
    p_obj = os.path.join(BUILD, "svdq_pack.o")
    _run([cxx] + HOST_FLAGS + ["-ffp-contract=off", "-c", os.path.join(CSRC, "svdq_pack.cpp"), "-o", p_obj])
    objs.append(p_obj)
    s_obj = os.path.join(BUILD, "svdq_svd.o")
    _run([cxx] + HOST_FLAGS + ["-march=x86-64-v3", "-ffp-contract=fast", "-c",
                               os.path.join(CSRC, "svdq_svd.cpp"), "-o", s_obj])
    objs.append(s_obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + ["-lpthread"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
