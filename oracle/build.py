"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so with g++.

The flags keep IEEE semantics: no FMA contraction, no fast-math, plain -O2.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gs_oracle.cpp")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-Werror", "-shared", "-fPIC", SRC, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
