"""Build libexpsketch.so in-tree for gfx950 with hipcc.

The sources compile to objects in parallel (the digit-organised update kernel,
the slowest to compile, once per instantiation), then link into one library.

Usage: python -m exp_density_sketching_amd.build   (or build() from Python)
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libexpsketch.so")

# (source, extra defines): one object each
UNITS = [("expsketch.hip", []), ("coreset.hip", [])] + [
    ("sk_update_kr.hip", [f"-DKR_RT={rt}", f"-DKR_CENTER={c}"])
    for rt in (1, 2, 4) for c in (0, 1)]
SOURCES = [os.path.join(CSRC, f) for f in sorted({u[0] for u in UNITS})]
HEADERS = [os.path.join(INCLUDE, "expsketch.h")] + [
    os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose=False):
    tmpdir = tempfile.mkdtemp(prefix="expsketch_build_")
    try:
        jobs = []
        for i, (src, defs) in enumerate(UNITS):
            obj = os.path.join(tmpdir, f"{i}_{os.path.splitext(src)[0]}.o")
            jobs.append(([HIPCC] + FLAGS + defs + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
        if verbose:
            for cmd, _ in jobs:
                print(" ".join(cmd), flush=True)
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            results = list(pool.map(lambda j: subprocess.run(j[0]), jobs))
        for (cmd, _), r in zip(jobs, results):
            if r.returncode != 0:
                raise subprocess.CalledProcessError(r.returncode, cmd)
        tmp = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for _, o in jobs] + ["-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
