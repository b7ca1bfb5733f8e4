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


# AddressSanitizer + UndefinedBehaviorSanitizer build (tests/test_sanitizers.py)
SANITIZE = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer"]


def build(verbose: bool = False, lib: str = LIB, sanitize: bool = False) -> str:
    tmp = lib + ".tmp"
    flags = [f for f in CFLAGS if not (sanitize and f == "-O2")] + (SANITIZE if sanitize else [])
    cmd = ["gcc", *flags, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
