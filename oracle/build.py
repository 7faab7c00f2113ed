"""Build the CPU oracle's shared library (test infrastructure only).

The oracle is plain C, compiled with value-safe floating point: no fused
multiply-add contraction and no fast-math, so every addition is one IEEE-754
binary32 operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "tide_oracle.c")
LIBRARY = os.path.join(HERE, "libtide_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-Werror",
        SOURCE, "-o", LIBRARY,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return LIBRARY


if __name__ == "__main__":
    print(build_oracle(verbose=True))
