"""Build librr.so (the HIP library behind include/rr.h) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librr.so")
SOURCES = [os.path.join(CSRC, "rr_ring.hip")]
HEADERS = [os.path.join(CSRC, "rr_device.hpp"), os.path.join(ROOT, "include", "rr.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 instructions stay off: hipcc would form them from plain float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every HIP source into ring_allreduce_amd/librr.so."""
    newest = max(os.path.getmtime(p) for p in SOURCES + HEADERS)
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= newest:
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
