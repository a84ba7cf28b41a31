"""Builds the CPU oracle, ``oracle/liboracle.so``, with g++.

Flags: -O3 without fast-math and with -ffp-contract=off, so every multiply and
add is rounded as written; x86-64-v3 (AVX2 + FMA) so the library built here
also runs on the GPU machine's host CPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

FLAGS = ["-O3", "-std=c++17", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
         "-fPIC", "-shared", "-pthread", "-fvisibility=hidden"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["g++", *FLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
