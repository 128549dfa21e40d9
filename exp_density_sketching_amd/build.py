"""Build libexpsketch.so in-tree for gfx950 with hipcc.

Usage: python -m exp_density_sketching_amd.build   (or build() from Python)
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libexpsketch.so")

SOURCES = [os.path.join(CSRC, "expsketch.hip")]
HEADERS = [os.path.join(INCLUDE, "expsketch.h")] + [
    os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
