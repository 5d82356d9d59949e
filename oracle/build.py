"""Builds the CPU oracle library with the host compiler (test infrastructure)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB_PATH = os.path.join(HERE, "liboracle.so")

# No FMA contraction and no fast-math: the oracle's double sums are exactly
# the written sequence of operations.
FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
         "-ffp-contract=off", "-fno-fast-math"]


def build_oracle(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = ["g++", *FLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_oracle(verbose=True))
