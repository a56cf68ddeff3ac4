"""Compile the CPU fp64 oracle (test infrastructure) into oracle/libg2oracle.so.

Plain C99 + OpenMP with gcc; nothing from the HIP library is compiled in.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "g2_oracle.c")
LIB = os.path.join(HERE, "libg2oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-shared", "-fPIC", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
