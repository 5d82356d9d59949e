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


SAN_MAIN = os.path.join(HERE, "sanitize_main.cpp")
SAN_BIN = os.path.join(os.path.dirname(HERE), "_build", "oracle_sanitized")


def build_sanitized(verbose: bool = False) -> str:
    """The oracle plus its driver (sanitize_main.cpp) as one host program under
    AddressSanitizer and UndefinedBehaviorSanitizer, every finding fatal.
    Host code only (g++; no GPU code is involved)."""
    os.makedirs(os.path.dirname(SAN_BIN), exist_ok=True)
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", SRC, SAN_MAIN, "-o", SAN_BIN]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return SAN_BIN


if __name__ == "__main__":
    print(build_oracle(verbose=True))
