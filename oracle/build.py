"""Build the CPU oracle library (plain C, gcc) next to its source.

TEST INFRASTRUCTURE ONLY (see moe_oracle.c).  Flags: no fast-math and no FMA
contraction, so every binary32/binary64 operation is the IEEE one written in
the source; OpenMP only splits independent tokens/rows across threads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
          "-fopenmp", "-fPIC", "-shared", "-Wall"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
