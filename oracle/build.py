"""Build the CPU oracle library (test infrastructure only).

Plain gcc, no fast-math and no FMA contraction, so every double operation in
qsa_oracle.c is rounded exactly as written.  OpenMP only splits independent
per-block and per-head loops; it changes no result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qsa_oracle.c")
LIB = os.path.join(HERE, "libqsa_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
