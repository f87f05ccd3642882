"""Compile ``workloads/libtreeopt.so`` (the contraction-tree search of
``treeopt.cpp``, host code only) with g++, in-tree."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "treeopt.cpp")
LIB = os.path.join(HERE, "libtreeopt.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-O3", "-march=x86-64-v2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-Wall", SRC,
           "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
