"""Compile the CPU oracle (plain C, gcc, OpenMP over rows) into oracle/liboracle.so.

Test infrastructure: the oracle is loaded only by the tests, the smoke check and
the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "graft_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
