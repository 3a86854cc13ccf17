"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so with g++.

The flags keep IEEE semantics: no FMA contraction, no fast-math, plain -O2.
build(sanitize=True) makes a checking build instead (AddressSanitizer and
UndefinedBehaviorSanitizer, aborting on the first report), for the CPU test job that
runs the oracle's pins under it (tests/test_oracle_sanitized.py); `python
oracle/build.py --sanitize` writes it to oracle/liboracle_san.so.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gs_oracle.cpp")
OUT = os.path.join(HERE, "liboracle.so")
OUT_SAN = os.path.join(HERE, "liboracle_san.so")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(verbose=False, sanitize=False, out=None):
    out = out or (OUT_SAN if sanitize else OUT)
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-Werror", "-shared", "-fPIC"] + (SANITIZE if sanitize else []) + [SRC, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def sanitizer_runtime():
    """Path of the AddressSanitizer runtime that a process loading the checking build
    must preload (the interpreter itself is not built with it)."""
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    return os.path.realpath(r.stdout.strip())


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv)
    sys.exit(0)
