"""allreduce_ring_staged_noalloc: the staged AllReduce for callers that cannot
allocate device memory, checked against allreduce_ring_staged (the entry point
it is a variant of) and the CPU oracle, bit for bit.

Its receive slots, signals and failure record live in a static device array of
the library, shared by every call on the device; the tests make calls in a row
with different sizes, check the size limits, a timed-out wait and the recovery
after it, and, in a fresh process, that a call changes no device-memory figure
while the allocating entry point's does."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import assert_matches_oracle, log, oracle_expect, to_host, to_slabs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DIST = {"int32": "int_pm1000", "fp32": "uniform_pm1", "bf16": "normal", "fp16": "normal"}
TORCH = {"int32": torch.int32, "fp32": torch.float32, "bf16": torch.bfloat16,
         "fp16": torch.float16}


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_allreduce_amd
    return ring_allreduce_amd


def _both(rr, x, dtype, op, ns, **opts):
    """The same inputs through both entry points; returns both outputs."""
    R, count = len(x), x[0].size
    send = to_slabs(rr, x, dtype, guard=True)
    out_a = [torch.full((count,), 3, dtype=TORCH[dtype], device="cuda") for _ in range(R)]
    out_b = [torch.full((count,), 5, dtype=TORCH[dtype], device="cuda") for _ in range(R)]
    rr.allreduce_ring_staged_noalloc(send.ranks, out_a, op, ns, **opts)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    rr.allreduce_ring_staged(send.ranks, out_b, op, ns, **opts)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    return [to_host(t, dtype) for t in out_a], [to_host(t, dtype) for t in out_b]


def test_two_calls_in_a_row_match_the_staged_loop(rr):
    """Two calls in a row, the second with a smaller input (fewer ranks, another
    dtype and op): each output equals allreduce_ring_staged's and the oracle's,
    bit for bit, on every element of every rank."""
    cases = [(8, 2_000_003, "fp32", "sum", 4), (5, 100_003, "bf16", "max", 3),
             (3, 40_001, "int32", "sum", 1)]
    for R, count, dtype, op, ns in cases:
        log(f"case noalloc R={R} count={count} {dtype} {op} ns={ns}")
        x = workloads.generate(R, count, dtype, DIST[dtype], 400 + R)
        got, ref = _both(rr, x, dtype, op, ns)
        assert_matches_oracle(got, ref, dtype, f"noalloc vs staged R={R}")
        assert_matches_oracle(got, oracle_expect(x, op), dtype, f"noalloc vs oracle R={R}")


def test_launch_per_step_and_single_rank(rr):
    """One launch per step (no signals) and R = 1 (a copy) through the static array."""
    x = workloads.generate(6, 33_333, "fp16", "normal", 41)
    got, ref = _both(rr, x, "fp16", "sum", 2, sync="launch")
    assert_matches_oracle(got, ref, "fp16", "noalloc launch per step")
    x1 = workloads.generate(1, 1001, "fp32", "uniform_pm1", 42)
    got, _ = _both(rr, x1, "fp32", "sum", 1)
    assert np.array_equal(got[0], x1[0].view(np.uint32))


def test_sizes_beyond_the_static_array_are_refused(rr):
    """Receive slots over 64 MiB, or more than 4096 (lane, rank) signal pairs:
    RR_ERR_UNSUPPORTED before anything is enqueued (the outputs keep their fill);
    the largest size that fits runs and matches."""
    R = 4
    big = (16 << 20) // 4 * R // 2 + 64       # fp32: 2 * R * chunk just over 64 MiB
    send = [torch.zeros(big, device="cuda") for _ in range(R)]
    recv = [torch.full((big,), 9.0, device="cuda") for _ in range(R)]
    st = rr.staged_ptrs("allreduce_noalloc", [t.data_ptr() for t in send],
                        [t.data_ptr() for t in recv], big, "fp32", "sum", 1)
    assert st == rr.RR_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert all(torch.all(t == 9.0) for t in recv)
    del send, recv
    # R * nslices > 4096 signal pairs
    send = [torch.zeros(64 * 256, device="cuda") for _ in range(64)]
    recv = [torch.zeros(64 * 256, device="cuda") for _ in range(64)]
    st = rr.staged_ptrs("allreduce_noalloc", [t.data_ptr() for t in send],
                        [t.data_ptr() for t in recv], 64 * 256, "fp32", "sum", 128)
    assert st == rr.RR_ERR_UNSUPPORTED
    del send, recv
    # the largest per-rank size at R = 4: 2 * 4 * chunk = 64 MiB exactly
    fit = (16 << 20) // 4 * R // 2
    x = workloads.generate(R, fit, "fp32", "uniform_pm1", 43)
    log(f"case noalloc largest R={R} count={fit}")
    got, ref = _both(rr, x, "fp32", "sum", 2)
    assert_matches_oracle(got, ref, "fp32", "noalloc at the limit")


def test_timeout_is_reported_and_cleared(rr):
    """A dropped arrival makes a wait time out: rr_last_kernel_error reports it
    from the static array's record and resets its signals, after which the next
    call is correct again."""
    x = workloads.generate(8, 8 * 4096 + 5, "fp32", "uniform_pm1", 44)
    send = to_slabs(rr, x, "fp32")
    recv = [torch.zeros(x[0].size, device="cuda") for _ in range(8)]
    rr.allreduce_ring_staged_noalloc(send.ranks, recv, "sum", 2,
                                     inject=rr.INJECT_DROP_ARRIVAL, timeout_ns=20_000_000)
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT and rec["expected"] - rec["observed"] >= 1
    assert rr.last_kernel_error()[0] == rr.RR_OK
    got, ref = _both(rr, x, "fp32", "sum", 2)
    assert_matches_oracle(got, ref, "fp32", "noalloc after a timeout")
    assert_matches_oracle(got, oracle_expect(x, "sum"), "fp32", "noalloc after a timeout")


_PROBE = r'''
import ctypes, sys
import torch
sys.path.insert(0, sys.argv[1])
import ring_allreduce_amd as rr
hip = ctypes.CDLL("libamdhip64.so.7")
hip.hipMemGetInfo.argtypes = [ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
def free():
    torch.cuda.synchronize()
    f, t = ctypes.c_size_t(), ctypes.c_size_t()
    assert hip.hipMemGetInfo(ctypes.byref(f), ctypes.byref(t)) == 0
    return f.value
R, small, large = 8, 4096, (3 << 20)
send = [torch.ones(large, device="cuda") for _ in range(R)]
recv = [torch.zeros(large, device="cuda") for _ in range(R)]
rr.allreduce_ring_staged_noalloc([t[:small] for t in send], [t[:small] for t in recv], "sum", 2)
rr.check_kernel_error()
f0 = free()
rr.allreduce_ring_staged_noalloc(send, recv, "sum", 2)
rr.check_kernel_error()
f1 = free()
assert torch.all(recv[0] == R).item()
rr.allreduce_ring_staged(send, recv, "sum", 2)
rr.check_kernel_error()
f2 = free()
print("noalloc", f0 - f1, "staged", f1 - f2, flush=True)
'''


def test_fresh_process_allocates_nothing():
    """In a fresh process: after a first small call (the library's code object,
    and with it the static array, is loaded then), a call with 12 MiB per rank
    leaves the device's free memory unchanged, while the allocating entry point
    on the same buffers takes at least its receive slots (2 x 12 MiB)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    run = subprocess.run([sys.executable, "-c", _PROBE, ROOT], capture_output=True, text=True,
                         timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    words = run.stdout.split()
    noalloc, staged = int(words[1]), int(words[3])
    assert noalloc == 0, run.stdout
    assert staged >= 2 * (12 << 20), run.stdout
