"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the
library, for the CPU test that runs the host ABI tests against it.

Only host code is instrumented: the HIP sources get the sanitizers through
-Xarch_host, the plain C++ sources are host-only; device code is built as
usual.  The result goes to _build/host_asan/libsvdq.so; the tests load it by
pointing SVDQ_LIBRARY at it, with clang's ASan runtime preloaded (Python
itself is not instrumented).  Run on the CPU only; it launches nothing."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "diffusion_smooth_group_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_asan")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
LIB = os.path.join(OUT, "libsvdq.so")

HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
COMMON = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include")]


def asan_runtime() -> str:
    cands = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not cands:
        raise FileNotFoundError("clang ASan runtime not found under ROCm's LLVM")
    return cands[-1]


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for name in ("svdq_kernels", "svdq_probe"):
        obj = os.path.join(OUT, name + ".o")
        cmd = [HIPCC, "--offload-arch=gfx950", "-ffp-contract=off"] + COMMON + HOST_SAN + \
              ["-c", os.path.join(CSRC, name + ".hip"), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True)
        objs.append(obj)
    for name, extra in (("svdq_pack", ["-ffp-contract=off"]), ("svdq_svd", ["-march=x86-64-v3"])):
        obj = os.path.join(OUT, name + ".o")
        cmd = [CLANGXX] + COMMON + extra + ["-fsanitize=address,undefined", "-D__HIP_PLATFORM_AMD__",
                                            "-I" + os.path.join(ROCM, "include"),
                                            "-c", os.path.join(CSRC, name + ".cpp"), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True)
        objs.append(obj)
    # linked by the host compiler (the HIP objects carry their device code
    # with them) against the HIP runtime
    cmd = [CLANGXX, "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address,undefined", "-o", LIB] + objs + \
          ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True)
    return LIB


def run_tests(pytest_args) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env["SVDQ_LIBRARY"] = LIB
    env["LD_PRELOAD"] = asan_runtime()
    # Python's own allocations are not instrumented: no leak report; stop at
    # the first error report of either sanitizer
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider"] + list(pytest_args),
                          cwd=ROOT, env=env, capture_output=True, text=True)


if __name__ == "__main__":
    build()
    r = run_tests(sys.argv[1:] or ["tests/test_lib_host.py"])
    print(r.stdout[-3000:], r.stderr[-3000:])
    sys.exit(r.returncode)
