"""Build the host backend of the input generator (libgen.so) with gcc.

Plain C99, -O2, OpenMP over counters.  Inputs only: the library draws the
workloads' seeded BF16 bits and computes nothing of the decode method.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gen.c")
LIB = os.path.join(HERE, "libgen.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
