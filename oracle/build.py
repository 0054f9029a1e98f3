"""Compile the fp64 CPU oracle (test infrastructure) into a shared library.

Usage: python oracle/build.py   (or oracle.build.build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cat_oracle.c")
LIB = os.path.join(HERE, "libcat_oracle.so")


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the library path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def needs_build() -> bool:
    return (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
