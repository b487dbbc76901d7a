"""Build the oracle's shared library (TEST INFRASTRUCTURE) with the host C compiler.

Plain ISO C99 at -O2 for one core: no intrinsics, no threads, no fast-math.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-Wall",
           "-Wextra", "-shared", "-fPIC", os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
