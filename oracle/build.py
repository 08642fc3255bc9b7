"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain C, gcc, optimisation -O2 with floating-point contraction off and no
fast-math, so float32 steps stay single IEEE operations."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q8s_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
