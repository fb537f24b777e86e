"""Builds oracle/liboracle.so with gcc (test infrastructure only).

-O2 with OpenMP over rows; no -ffast-math and -ffp-contract=off, so that
every float operation is the one written in the source.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qsa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
