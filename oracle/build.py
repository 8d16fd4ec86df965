"""Build the CPU oracle (TEST INFRASTRUCTURE) into oracle/liboracle.so with gcc.

Plain C99, -O2 with loop vectorisation but no fast-math and no FMA contraction
(the oracle's arithmetic stays IEEE fp64, in the order the source states),
OpenMP over rows / heads.  Run as `python oracle/build.py`.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "ncgpt_oracle.c"), os.path.join(HERE, "optim_oracle.c")]
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-ftree-vectorize", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", OUT + ".tmp", *SRCS, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
