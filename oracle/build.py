"""Build the host oracle library (``liboracle.so``) with gcc.

Test infrastructure: plain C, OpenMP over rows, no fast-math, no
floating-point contraction.  Shares nothing with the GPU library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CMD = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
       "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB, SRC, "-lm"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = CMD[:-3] + [tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
