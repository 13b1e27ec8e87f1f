"""Compile the C oracle (dsa_oracle.c) into oracle/libdsa_oracle.so with gcc.

Strict IEEE fp64: no fast-math, no FMA contraction, so every sum is the plain
left-to-right loop written in the source.  Test infrastructure only.
"""
import os
import subprocess

ORACLE_DIR = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(ORACLE_DIR, "dsa_oracle.c")
ORACLE_LIB = os.path.join(ORACLE_DIR, "libdsa_oracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def build_oracle(verbose=False):
    tmp = ORACLE_LIB + ".tmp"
    cmd = ["gcc"] + GCC_FLAGS + [ORACLE_SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, ORACLE_LIB)
    return ORACLE_LIB


if __name__ == "__main__":
    build_oracle(verbose=True)
