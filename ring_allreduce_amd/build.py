"""Build librr.so (the HIP library behind include/rr.h) for gfx950, in-tree."""
from __future__ import annotations

import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librr.so")
# one translation unit per kernel family (the in-place ring: one per element
# type), and the host side with the C ABI
SOURCES = [os.path.join(CSRC, f) for f in
           ("rr_ring_i32.hip", "rr_ring_f32.hip", "rr_ring_bf16.hip", "rr_ring_f16.hip",
            "rr_staged_kernel.hip", "rr_aux_kernels.hip", "rr_api.hip")]
HEADERS = [os.path.join(CSRC, "rr_device.hpp"), os.path.join(CSRC, "rr_kernels.hpp"),
           os.path.join(CSRC, "rr_ring_kernel.hpp"), os.path.join(ROOT, "include", "rr.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions stay off: hipcc would form them from plain float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def declared_functions() -> list[str]:
    """The functions include/rr.h declares: the library's whole dynamic interface."""
    with open(os.path.join(ROOT, "include", "rr.h")) as fh:
        text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
    decl = re.compile(r"^(?:const\s+)?\w+[\s*]+(\w+)\s*\(", re.M)
    return sorted(set(decl.findall(text)))


def _version_script(path: str) -> str:
    """Export the declared functions only; kernel handles and helpers stay local."""
    with open(path, "w") as fh:
        fh.write("{\n  global:\n")
        fh.writelines("    %s;\n" % name for name in declared_functions())
        fh.write("  local: *;\n};\n")
    return path


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link ring_allreduce_amd/librr.so."""
    newest = max(os.path.getmtime(p) for p in SOURCES + HEADERS)
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= newest:
        return LIB
    include = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="rr_build_") as tmpdir:
        objects = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]

        def compile_one(job):
            src, obj = job
            cmd = [HIPCC, *FLAGS, *include, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
            list(pool.map(compile_one, zip(SOURCES, objects)))
        tmp = LIB + ".tmp%d" % os.getpid()
        script = _version_script(os.path.join(tmpdir, "exports.map"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
               "-Wl,--version-script=" + script, "-o", tmp, *objects]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
