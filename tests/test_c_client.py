"""The C ABI from plain C.

include/rr.h must compile as C99 with -Wall -Wextra -Werror -pedantic; a C
program linked against librr.so must get the answers the header documents for
calls decided on the host (argument checks, no-ops, status strings); and the
size and field offsets of every struct the header declares must be the ones the
Python binding's ctypes structures use.  On a GPU, a second C program runs the
ring itself through the C ABI (no Python in between) and checks the results
against the definition."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    import ring_allreduce_amd
    lib_dir = os.path.dirname(ring_allreduce_amd.LIB_PATH)
    exe = str(tmp_path_factory.mktemp("c_client") / "abi_client")
    build = subprocess.run(
        [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
         "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c", "abi_client.c"),
         "-o", exe, "-L", lib_dir, "-lrr", "-Wl,-rpath," + lib_dir],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    return ring_allreduce_amd, run


def test_c_client_gets_the_documented_host_answers(client):
    _, run = client
    assert run.returncode == 0, run.stderr
    assert run.stdout.strip().splitlines()[-1] == "ok"


@pytest.mark.parametrize("c_name,py_name", [("rr_options_t", "Options"), ("rr_plan_t", "_Plan"),
                                            ("rr_error_record_t", "ErrorRecord")])
def test_struct_layouts_match_the_binding(client, c_name, py_name):
    rr, run = client
    line = next(l for l in run.stdout.splitlines() if l.startswith(c_name + " "))
    seen = dict((k, int(v)) for k, v in re.findall(r"(\w+)=(\d+)", line))
    cls = getattr(rr, py_name)
    assert seen.pop("size") == ctypes.sizeof(cls)
    py = {name: getattr(cls, name).offset for name, _ in cls._fields_}
    assert seen == py


def _build_gpu_client(out_dir):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    import ring_allreduce_amd
    lib_dir = os.path.dirname(ring_allreduce_amd.LIB_PATH)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(out_dir / "gpu_client")
    build = subprocess.run(
        [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
         "-isystem", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
         os.path.join(HERE, "c", "gpu_client.c"), "-o", exe,
         "-L", lib_dir, "-lrr", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
         "-Wl,-rpath," + lib_dir, "-Wl,-rpath," + os.path.join(rocm, "lib")],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    return exe


def test_gpu_client_compiles_as_c99(tmp_path):
    _build_gpu_client(tmp_path)


@pytest.mark.gpu
def test_gpu_client_runs_the_ring(tmp_path):
    """SUM with predecessor hand-offs and MAX with a counting barrier, 8 ranks of
    int32 in separate allocations, checked element by element against the
    definition by the C program itself."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = _build_gpu_client(tmp_path)
    print("case C client: R=8 int32 SUM p2p and MAX barrier", flush=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip().splitlines()[-1] == "ok"
