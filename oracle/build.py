"""Compile the C part of the CPU oracle (test infrastructure only).

``python -m oracle.build`` or :func:`build` writes ``oracle/libnvfp4_ref.so``
with gcc: -O2, OpenMP over independent rows, no fast-math and no floating-point
contraction, so every row is summed exactly as ``nvfp4_ref.c`` is written.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_ref.c")
LIB = os.path.join(HERE, "libnvfp4_ref.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
