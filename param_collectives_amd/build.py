"""Compile the HIP library (libtide.so) for gfx950, in-tree.

Flags that matter for results:
  -ffp-contract=off    no fused multiply-add contraction anywhere;
  no -ffast-math / -fgpu-flush-denormals-to-zero: fp32 subnormals are kept;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                       the compiler emits no packed-fp32 VALU instructions.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libtide.so")
SOURCES = [os.path.join(CSRC, n) for n in ("plan.cpp", "capi.cpp", "kernels.hip", "instruments.hip", "scratch.hip")]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build_library(verbose: bool = False, extra=()) -> str:
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        *SOURCES, "-o", LIBRARY + ".tmp",
        *extra,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build_library(verbose=True))
