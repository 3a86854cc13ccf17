"""Build libgs.so (the HIP library behind include/gs.h) for gfx950 with hipcc.

Every translation unit is compiled separately so that the projection unit can be
built without floating-point contraction (its key path must be plain IEEE fp32).
Packed-fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libgs.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["preprocess.hip", "chain.hip", "scan.hip", "sort.hip", "render.hip", "loss.hip", "adam.hip", "layout.hip",
           "densify.hip", "profile.hip", "gs_api.hip"]
PER_FILE_FLAGS = {"preprocess.hip": ["-ffp-contract=off"], "chain.hip": ["-ffp-contract=off"],
                  "densify.hip": ["-ffp-contract=off"]}
ARCH = os.environ.get("GS_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics",
            "-Wall", "-Wno-unused-function", "-Werror"]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + common_flags() + PER_FILE_FLAGS.get(src, [])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose=False, jobs=8):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(OUT)
