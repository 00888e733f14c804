"""Build the fp64 Soft-DTW oracle (test infrastructure only) with gcc.

Produces ``oracle/libsdtw_oracle.so`` beside this file.  The oracle is plain
C with OpenMP over the batch; it is compiled without fast-math and without
floating-point contraction so every operation rounds as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sdtw_oracle.c")
LIB = os.path.join(HERE, "libsdtw_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-shared", "-fPIC", "-Wall", "-Wextra",
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
