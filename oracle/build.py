"""Compile the C oracle (kda_ref_cpu.c) into oracle/libkda_ref.so.

Test infrastructure: building the checker is not using it.  Plain -O2 with
OpenMP and the baseline x86-64 instruction set, so the library built here
also runs on other hosts.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_ref_cpu.c")
LIB = os.path.join(HERE, "libkda_ref.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
