"""Compile the CPU oracle (rnn_oracle.c) into oracle/librnn_oracle.so.

The oracle is test infrastructure: plain C, binary32 arithmetic with no
contraction (-ffp-contract=off) and no fast-math, OpenMP threads over
independent rows only (each output keeps its own sequential accumulator, so
the result does not depend on the thread count).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rnn_oracle.c")
LIB = os.path.join(HERE, "librnn_oracle.so")

CFLAGS = ["-std=c11", "-O3", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
