"""Workspace lifecycle: rr_finalize frees every device's workspace and the staged
loop's receive buffers, and the next call creates them afresh; results before
and after match the CPU oracle bit for bit, and a failure record from before
does not survive."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_matches_oracle, log, oracle_expect, to_device, to_host, to_slabs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_allreduce_amd
    ring_allreduce_amd.init()
    return ring_allreduce_amd


def _every_collective(rr, x, expect):
    s = to_slabs(rr, x, "fp32")
    rr.allreduce_ring(s.ranks, "sum", 2, sync="barrier")
    t = to_slabs(rr, x, "fp32")
    recv = rr.allreduce_ring_staged(t.ranks, None, "sum", 2)
    R, n = len(x), x[0].size
    send = [to_device(a, "fp32") for a in x]
    out = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(R)]
    rr.alltoall(send, out)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert_matches_oracle([to_host(r_, "fp32") for r_ in s.ranks], expect, "fp32", "ring")
    assert_matches_oracle([to_host(r_, "fp32") for r_ in recv], expect, "fp32", "staged")
    want = [w.view(np.uint32) for w in oracle.alltoall(x)]
    assert_matches_oracle([to_host(o, "fp32") for o in out], want, "fp32", "alltoall")


def test_finalize_then_call_again(rr):
    R, n = 8, 8 * 6000      # alltoall blocks of 6000 elements
    x = workloads.generate(R, n, "fp32", "uniform_pm1", 61)
    expect = oracle_expect(x, "sum")
    for k in range(3):
        log(f"case lifecycle pass {k}")
        _every_collective(rr, x, expect)
        rr.finalize()
    rr.init()
    _every_collective(rr, x, expect)


def test_failure_record_does_not_survive_finalize(rr):
    """A timed-out wait leaves a sticky record (later calls return at once while it
    stands).  Left unread, it is dropped with the workspace by rr_finalize: the
    next call runs on a clean workspace and reports no error."""
    R, n = 8, 8 * 20000 + 3
    x = workloads.generate(R, n, "fp32", "uniform_pm1", 62)
    s = to_slabs(rr, x, "fp32")
    log("case lifecycle: injected missing arrival, record left unread, finalize")
    rr.allreduce_ring(s.ranks, "sum", 4, sync="p2p", inject=rr.INJECT_DROP_ARRIVAL,
                      timeout_ns=20_000_000)
    torch.cuda.synchronize()
    rr.finalize()
    s = to_slabs(rr, x, "fp32")
    rr.allreduce_ring(s.ranks, "sum", 4, sync="p2p")
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert_matches_oracle([to_host(t, "fp32") for t in s.ranks], oracle_expect(x, "sum"),
                          "fp32", "after finalize")
