"""The C-ABI library: it loads, exports what include/rr.h declares, and rejects
bad arguments on the host before touching a device (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rr.h")


@pytest.fixture(scope="module")
def rr():
    import ring_allreduce_amd
    return ring_allreduce_amd


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\**\s*([a-z_][a-z_0-9]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ["allreduce_ring", "reduce_scatter_ring", "all_gather_ring",
                     "counting_barrier_create", "counting_barrier_run", "counting_barrier_read",
                     "counting_barrier_reset", "counting_barrier_destroy",
                     "rr_last_kernel_error"]:
        assert required in names


def test_library_exports_nothing_but_the_header(rr):
    """The dynamic interface is exactly what include/rr.h declares: kernel handles and
    internal helpers of the library stay local."""
    out = subprocess.run(["nm", "-D", "--defined-only", rr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines())
    assert exported == _declared_functions()


def test_library_exports_every_declared_symbol(rr):
    names = _declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", rr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(rr.EXPORTED) == names
    lib = ctypes.CDLL(rr.LIB_PATH)
    for n in names:
        assert hasattr(lib, n)


def test_abi_version_and_status_strings(rr):
    assert rr.abi_version() == 1
    for code, name in rr.STATUS.items():
        assert rr.status_string(code).startswith(name)
    assert "unknown" in rr.status_string(99)


A = 0x7F0000000000  # 16-byte aligned addresses; never dereferenced by these tests


@pytest.mark.parametrize("case", [
    dict(ptrs=[], count=16),                                    # R = 0
    dict(ptrs=[A + i * 4096 for i in range(65)], count=16),     # R = 65
    dict(ptrs=[A, A + 4096], count=16, nslices=0),
    dict(ptrs=[A, A + 4096], count=16, nslices=1025),
    dict(ptrs=[A, A + 4096], count=16, dtype=7),
    dict(ptrs=[A, A + 4096], count=16, op=5),
    dict(ptrs=[A, A + 4104], count=16),                         # misaligned
    dict(ptrs=[A, 0], count=16),                                # null buffer
    dict(ptrs=[A, A + 32], count=16),                           # overlap (64 bytes each)
    dict(ptrs=[A + 4096, A, A + 4096 + 16], count=8),           # overlap after sorting
    dict(ptrs=[A, A + 4096], count=16, sync=9),
    dict(ptrs=[A, A + 4096], count=16, sync="per_peer"),   # barrier runs only
    dict(ptrs=[A, A + 4096], count=16, block=192),
    dict(ptrs=[A, A + 4096], count=16, team=-1),
    dict(ptrs=[A, A + 4096], count=16, rounds=-1),
    dict(ptrs=[A, A + 4096], count=16, depth=5),
    dict(ptrs=[A, A + 4096], count=(1 << 40) + 1),
])
def test_invalid_arguments_rejected_on_host(rr, case):
    kw = dict(case)
    ptrs = kw.pop("ptrs")
    count = kw.pop("count")
    st = rr.allreduce_ring_ptrs(ptrs, count, kw.pop("dtype", "fp32"), kw.pop("op", "sum"),
                                kw.pop("nslices", 1), **kw)
    assert st == rr.RR_ERR_INVALID


B = A + (1 << 30)  # a second region, far from the first


@pytest.mark.parametrize("kind", ["allreduce", "reduce_scatter", "all_gather", "alltoall"])
@pytest.mark.parametrize("case", [
    dict(send=[], recv=[], n=16),                                              # R = 0
    dict(send=[A + i * 4096 for i in range(65)], recv=[B + i * 4096 for i in range(65)], n=16),
    dict(send=None, recv=[B, B + 4096], n=16),
    dict(send=[A, A + 4096], recv=None, n=16),
    dict(send=[A, 0], recv=[B, B + 4096], n=16),
    dict(send=[A, A + 4096], recv=[B, B + 8], n=16),                           # misaligned
    dict(send=[A, A + 32], recv=[B, B + 4096], n=16),                          # sends overlap
    dict(send=[A, A + 4096], recv=[A + 4096 + 16, B], n=16),                   # recv overlaps a send
    dict(send=[A, A + 4096], recv=[B, B + 4096], n=16, dtype=9),
    dict(send=[A, A + 4096], recv=[B, B + 4096], n=16, op=9),
    dict(send=[A, A + 4096], recv=[B, B + 4096], n=16, nslices=0),
    dict(send=[A, A + 4096], recv=[B, B + 4096], n=16, sync=9),
    dict(send=[A, A + 4096], recv=[B, B + 4096], n=16, rounds=-1),
    dict(send=[A, A + 4096], recv=[B, B + 4096], n=(1 << 40) + 1),
])
def test_staged_invalid_arguments(rr, kind, case):
    if kind in ("all_gather", "alltoall") and "op" in case:
        pytest.skip(f"{kind} takes no op")
    if kind == "alltoall" and ("nslices" in case or "rounds" in case):
        pytest.skip("alltoall takes no slices or rounds")
    kw = dict(case)
    st = rr.staged_ptrs(kind, kw.pop("send"), kw.pop("recv"), kw.pop("n"), kw.pop("dtype", "fp32"),
                        kw.pop("op", "sum"), kw.pop("nslices", 1), **kw)
    assert st == rr.RR_ERR_INVALID


def test_staged_in_place_rules(rr):
    """An AllReduce may receive in place; the standalone collectives may not."""
    assert rr.staged_ptrs("allreduce", [A, A + 4096], [A, A + 4096], 0, "fp32") == rr.RR_OK
    same = [A, A + (1 << 20)]
    assert rr.staged_ptrs("reduce_scatter", same, same, 16, "fp32") == rr.RR_ERR_INVALID
    assert rr.staged_ptrs("all_gather", same, same, 16, "fp32") == rr.RR_ERR_INVALID
    # a receive buffer may not be another rank's send buffer, even in an AllReduce
    assert rr.staged_ptrs("allreduce", [A, A + 4096], [A + 4096, A], 16, "fp32") == \
        rr.RR_ERR_INVALID


def test_null_buffer_array(rr):
    st = rr._allreduce_ring(None, 4, 16, 1, 0, 1, None)
    assert st == rr.RR_ERR_INVALID


@pytest.mark.parametrize("phase", ["reduce_scatter", "all_gather"])
def test_invalid_arguments_other_phases(rr, phase):
    st = rr.allreduce_ring_ptrs([A, A + 8], 16, "fp32", "sum", 1, phase=phase)
    assert st == rr.RR_ERR_INVALID


def test_trivial_calls_are_no_ops(rr):
    # one rank, or nothing to reduce: success without any device work
    assert rr.allreduce_ring_ptrs([A], 1 << 20, "fp32") == rr.RR_OK
    assert rr.allreduce_ring_ptrs([A, A + 4096], 0, "bf16") == rr.RR_OK


def test_counting_barrier_rejects_bad_shapes(rr):
    h = ctypes.c_void_p()
    assert rr._cb_create(0, 1, ctypes.byref(h)) == rr.RR_ERR_INVALID
    assert rr._cb_create(65, 1, ctypes.byref(h)) == rr.RR_ERR_INVALID
    assert rr._cb_create(4, 0, ctypes.byref(h)) == rr.RR_ERR_INVALID
    assert rr._cb_create(4, 1025, ctypes.byref(h)) == rr.RR_ERR_INVALID
    assert rr._cb_create(4, 1, None) == rr.RR_ERR_INVALID
    assert rr._cb_destroy(None) == rr.RR_OK
    assert rr._cb_run(None, 4, 1, 1, 3, None, None) == rr.RR_ERR_INVALID
    n = ctypes.c_uint64()
    assert rr._cb_read_peer(None, 0, 0, 1, ctypes.byref(n), ctypes.byref(n)) == rr.RR_ERR_INVALID
    assert rr._cb_early(None, 0, 0, ctypes.byref(n)) == rr.RR_ERR_INVALID


def test_copy_rejects_bad_arguments(rr):
    assert rr._hbm_copy(None, A, 16, None) == rr.RR_ERR_INVALID
    assert rr._hbm_copy(A + 8, A + 4096, 16, None) == rr.RR_ERR_INVALID
    assert rr._hbm_copy(A, A + 8, 64, None) in (rr.RR_ERR_INVALID,)
    assert rr._hbm_copy(A, A + 4096, 0, None) == rr.RR_OK


def test_plan_query_rejects_bad_arguments(rr):
    p = rr._Plan()
    assert rr._plan_query(0, 16, 1, 1, 0, None, ctypes.byref(p)) == rr.RR_ERR_INVALID
    assert rr._plan_query(4, 16, 1, 1, 7, None, ctypes.byref(p)) == rr.RR_ERR_INVALID
    assert rr._plan_query(4, 16, 4, 1, 0, None, ctypes.byref(p)) == rr.RR_ERR_INVALID
    assert rr._plan_query(4, 16, 1, 1, 0, None, None) == rr.RR_ERR_INVALID


def test_product_path_has_no_oracle_dependency():
    """The GPU library and its binding never reach into the oracle."""
    pkg = os.path.join(ROOT, "ring_allreduce_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.lower(), f
    out = subprocess.run(["ldd", os.path.join(pkg, "librr.so")], capture_output=True, text=True).stdout
    assert "ring_oracle" not in out


@pytest.mark.parametrize("phase,opts", [
    (0, dict(team=4097)), (0, dict(rounds=5000)), (0, dict(depth=5)), (0, dict(block=192)),
    (0, dict(sync=4)), (2, dict(team=-1)), (3, dict(team=4097)), (4, dict(rounds=-1)),
    (5, dict(block=96)), (6, dict(sync=2)), (6, dict(team=65537)),
    (0, dict(flags=0x80 | 0x800)), (1, dict(flags=0x100 | 0x400)), (2, dict(flags=0x200 | 0x100)),
    (0, dict(flags=0x1000 | 0x2000)), (1, dict(order="ascending", flags=0x2000)),
])
def test_plan_query_rejects_what_the_call_rejects(rr, phase, opts):
    """The plan query checks options and sizes as the calls do, before any
    device work (so the same argument never passes one and fails the other)."""
    p = rr._Plan()
    o = rr._options(**opts)
    assert rr._plan_query(4, 1 << 20, 1, 1, phase, ctypes.byref(o), ctypes.byref(p)) == \
        rr.RR_ERR_INVALID


@pytest.mark.parametrize("phase", [3, 4, 5, 6])
def test_plan_query_rejects_oversized_block_sets(rr, phase):
    p = rr._Plan()
    assert rr._plan_query(8, (1 << 40) // 4, 1, 1, phase, None, ctypes.byref(p)) == \
        rr.RR_ERR_INVALID


def test_build_script_loads_without_the_library():
    """build() must work in a fresh checkout, where librr.so does not exist yet:
    it loads the build script by path, without running the package's __init__
    (which refuses to import until the library is built)."""
    code = ("import sys, __graft_entry__ as g; m = g._load_build_script(); "
            "assert callable(m.build) and m.LIB.endswith('librr.so'); "
            "assert 'ring_allreduce_amd' not in sys.modules")
    subprocess.run([os.sys.executable, "-c", code], cwd=ROOT, check=True)


def test_timed_barrier_run_validates_on_host(rr):
    """counting_barrier_run_timed rejects a missing object, stamps buffer or
    clock out-pointer before any device work."""
    khz = ctypes.c_uint32()
    assert rr._cb_run_timed(None, 2, 1, 1, 1, None, A, ctypes.byref(khz), None) == \
        rr.RR_ERR_INVALID
    fake = ctypes.c_void_p(A)
    assert rr._cb_run_timed(fake, 2, 1, 1, 1, None, None, ctypes.byref(khz), None) == \
        rr.RR_ERR_INVALID
    assert rr._cb_run_timed(fake, 2, 1, 1, 1, None, A, None, None) == rr.RR_ERR_INVALID


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with a message and status 2."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    run = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=root)
    assert run.returncode == 2
    assert "one GPU" in run.stdout + run.stderr
