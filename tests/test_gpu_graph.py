"""The collectives captured in a HIP graph and replayed.

Every replay must match the CPU oracle bit for bit, with eager calls of the
library between the replays and the program's own synchronisations around them.
A replay re-runs a launch with its captured arguments, so nothing a kernel needs
to tell one launch from the next may come from the host: the per-launch tag of
the XCD table lives on the device and the last workgroup of every launch
advances it (otherwise a replayed launch could take the previous launch's table
entries for its own).  Inputs are restored eagerly before each replay; the
graphs hold kernel launches only (no memset nodes)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import (assert_matches_oracle, log, oracle_expect, to_device, to_host,
                            to_slabs)

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_allreduce_amd
    ring_allreduce_amd.init()
    return ring_allreduce_amd


def _capture(fn):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _other_work(rr):
    """An eager call of another collective between replays (it advances the
    device-side launch tag and leaves its own XCD table entries behind)."""
    x = workloads.generate(16, 4096 + 7, "int32", "int_pm1000", 77)
    s = to_slabs(rr, x, "int32", guard=False)
    rr.allreduce_ring(s.ranks, "sum", 2, sync="barrier")
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert_matches_oracle([to_host(t, "int32") for t in s.ranks], oracle_expect(x, "sum"),
                          "int32", "eager call between replays")


def _replay_and_check(rr, g, restore, read, expect, dtype, what):
    for k in range(REPLAYS):
        restore()
        _other_work(rr)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rr.check_kernel_error()
        assert_matches_oracle(read(), expect, dtype, f"{what}, replay {k}")


@pytest.mark.parametrize("R,count,dtype,op,ns,sync,flags", [
    (8, 3 * 4096 + 5, "fp32", "sum", 4, "p2p", 0),
    (16, 65536 + 3, "bf16", "sum", 2, "barrier", 0),
    (4, 1000, "int32", "max", 1, "launch", 0),           # one launch per hop: 6 kernels
    (8, 1 << 16, "fp32", "sum", 4, "p2p", "fused"),
    (64, 8 * 1024 + 4, "fp32", "sum", 8, "barrier", 0),
    (16, 65536 + 3, "fp32", "sum", 4, "barrier", "alternate"),  # the alternating kernel
    (4, 1000, "bf16", "sum", 1, "launch", "alternate"),          # ... one launch per hop
])
def test_ring_allreduce_replays(rr, R, count, dtype, op, ns, sync, flags):
    log(f"case graph ring R={R} count={count} {dtype} {op} ns={ns} sync={sync} flags={flags}")
    x = workloads.generate(R, count, dtype, "normal" if dtype == "bf16" else
                           ("int_pm1000" if dtype == "int32" else "uniform_pm1"), 31 + R)
    expect = oracle_expect(x, op)
    slabs = to_slabs(rr, x, dtype)
    pristine = slabs.storage.clone()
    opts = dict(sync=sync)
    if flags == "fused":
        opts["fused"] = True
    elif flags == "alternate":
        opts["order"] = "alternate"

    def call():
        rr.allreduce_ring(slabs.ranks, op, ns, **opts)

    call()                                   # eager, on the pristine inputs
    torch.cuda.synchronize()
    rr.check_kernel_error()
    read = lambda: [to_host(t, dtype) for t in slabs.ranks]
    assert_matches_oracle(read(), expect, dtype, "eager")
    slabs.storage.copy_(pristine)
    g = _capture(call)
    _replay_and_check(rr, g, lambda: slabs.storage.copy_(pristine), read, expect, dtype,
                      "ring replay")


def test_reduce_scatter_then_all_gather_in_one_graph(rr):
    R, count, dtype = 8, 8 * 1024 + 12, "fp32"
    log(f"case graph rs+ag R={R} count={count}")
    x = workloads.generate(R, count, dtype, "uniform_pm1", 5)
    expect = oracle_expect(x, "sum")
    slabs = to_slabs(rr, x, dtype)
    pristine = slabs.storage.clone()

    def call():
        rr.reduce_scatter_ring(slabs.ranks, "sum", 2)
        rr.all_gather_ring(slabs.ranks, 2)

    g = _capture(call)
    _replay_and_check(rr, g, lambda: slabs.storage.copy_(pristine),
                      lambda: [to_host(t, dtype) for t in slabs.ranks], expect, dtype,
                      "rs+ag replay")


def test_staged_allreduce_replays(rr):
    R, count, dtype = 8, 4 * 8192 + 3, "fp32"
    log(f"case graph staged R={R} count={count}")
    x = workloads.generate(R, count, dtype, "uniform_pm1", 6)
    expect = oracle_expect(x, "sum")
    send = to_slabs(rr, x, dtype)
    recv = [torch.empty(count, dtype=torch.float32, device="cuda") for _ in range(R)]

    def call():
        rr.allreduce_ring_staged(send.ranks, recv, "sum", 4)

    call()                                   # eager: allocates the receive slots
    torch.cuda.synchronize()
    rr.check_kernel_error()
    g = _capture(call)

    def clear():
        for t in recv:
            t.fill_(-1.0)

    _replay_and_check(rr, g, clear, lambda: [to_host(t, dtype) for t in recv], expect, dtype,
                      "staged replay")
    for r in range(R):                       # out of place: the inputs are untouched
        assert np.array_equal(to_host(send.ranks[r], dtype), x[r].view(np.uint32))


def test_alltoall_replays(rr):
    R, n, dtype = 8, 4099, "bf16"
    log(f"case graph alltoall R={R} n={n}")
    x = workloads.generate(R, R * n, dtype, "normal", 8)
    send = [to_device(a, dtype) for a in x]
    recv = [torch.empty(R * n, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    want = [w.view(np.uint16) for w in oracle.alltoall(x)]

    def call():
        rr.alltoall(send, recv)

    call()
    torch.cuda.synchronize()
    rr.check_kernel_error()
    g = _capture(call)

    def clear():
        for t in recv:
            t.zero_()

    _replay_and_check(rr, g, clear, lambda: [to_host(t, dtype) for t in recv], want, dtype,
                      "alltoall replay")


def test_staged_replay_after_the_receive_buffers_grew(rr):
    """A staged call captured while the receive buffers were small, replayed
    after a larger eager call grew them (and after allocations that could have
    taken the old buffers' memory): the replay still writes into buffers it
    owns and matches the oracle, because outgrown receive buffers are kept until
    rr_finalize."""
    R, count, dtype = 8, 4 * 8192 + 3, "fp32"
    log(f"case graph staged after growth R={R} count={count}")
    rr.finalize()                            # start from no receive buffers at all
    rr.init()
    x = workloads.generate(R, count, dtype, "uniform_pm1", 16)
    expect = oracle_expect(x, "sum")
    send = to_slabs(rr, x, dtype)
    recv = [torch.empty(count, dtype=torch.float32, device="cuda") for _ in range(R)]

    def call():
        rr.allreduce_ring_staged(send.ranks, recv, "sum", 4)

    call()                                   # eager: receive buffers for this size
    torch.cuda.synchronize()
    rr.check_kernel_error()
    g = _capture(call)
    big_n = 16 * count
    xb = workloads.generate(R, big_n, dtype, "uniform_pm1", 17)
    big_send = to_slabs(rr, xb, dtype)
    big_recv = rr.allreduce_ring_staged(big_send.ranks, None, "sum", 4)  # grows them
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert_matches_oracle([to_host(t, dtype) for t in big_recv], oracle_expect(xb, "sum"), dtype,
                          "the larger eager call")
    del big_send, big_recv
    fillers = [torch.full((count,), 7.0, device="cuda") for _ in range(4 * R)]

    def clear():
        for t in recv:
            t.fill_(-1.0)

    _replay_and_check(rr, g, clear, lambda: [to_host(t, dtype) for t in recv], expect, dtype,
                      "staged replay after growth")
    for t in fillers:                        # nothing wrote into other allocations
        assert torch.all(t == 7.0)
