"""GPU tests of the signal layer: the standalone counting barrier, the rolling
comparison near 2^64, and the bounded waits (timeouts forced from the host by an
unsatisfiable expectation with a short limit, so every workgroup still exits)."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import assert_matches_oracle, log, oracle_expect, to_host, to_slabs

pytestmark = pytest.mark.gpu

SHORT = 20_000_000  # 20 ms wait limit for the forced timeouts


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_allreduce_amd
    ring_allreduce_amd.init()
    st, _ = ring_allreduce_amd.last_kernel_error()  # start from a clear record
    return ring_allreduce_amd


@pytest.mark.parametrize("R,nctx,mode", [(2, 1, "barrier"), (8, 4, "barrier"), (64, 8, "barrier"),
                                        (16, 2, "p2p"), (64, 1, "p2p")])
def test_counting_barrier_counts(rr, R, nctx, mode):
    log(f"case barrier counts R={R} nctx={nctx} mode={mode}")
    b = rr.CountingBarrier(64, 8)
    steps = 50
    b.run(R, steps, nctx, mode=mode)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    per = (R - 1) if mode == "barrier" else 1
    for ctx in range(nctx):
        for waiter in (0, R // 2, R - 1):
            v, s = b.read(ctx, waiter)
            assert v == s == steps * per
    # untouched context and waiters stay at zero
    if nctx < 8:
        assert b.read(nctx, 0) == (0, 0)
    if R < 64:
        assert b.read(0, R) == (0, 0)
    b.run(R, 7, nctx, mode=mode)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert b.read(0, 0) == (57 * per, 57 * per)
    b.close()


def test_counting_barrier_wraps(rr):
    log("case barrier wrap")
    b = rr.CountingBarrier(8, 1)
    start = (1 << 64) - 5
    b.preset(start)
    b.run(8, 10, 1)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    v, s = b.read(0, 3)
    assert v == s == (start + 70) % (1 << 64)
    b.reset()
    assert b.read(0, 3) == (0, 0)
    b.close()


def test_counting_barrier_zero_steps(rr):
    b = rr.CountingBarrier(4, 1)
    b.run(4, 0, 1)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert b.read(0, 0) == (0, 0)
    b.close()


def test_counting_barrier_missing_arrival_times_out(rr):
    """An expectation one above what arrives: the waiter gives up and reports it."""
    log("case barrier timeout")
    b = rr.CountingBarrier(8, 2)
    b.run(8, 5, 2, expected=8, timeout_ns=SHORT)  # R-1 = 7 arrive per step
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT
    assert rec["expected"] - rec["observed"] == 1 and rec["hop"] == 1
    assert rr.last_kernel_error()[0] == rr.RR_OK  # reading cleared it
    b.reset()
    b.run(8, 5, 2)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert b.read(1, 7) == (35, 35)
    b.close()


def test_counting_barrier_injected_drop(rr):
    log("case barrier drop")
    b = rr.CountingBarrier(4, 1)
    b.run(4, 3, 1, inject=rr.INJECT_DROP_ARRIVAL, timeout_ns=SHORT)
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT and rec["expected"] - rec["observed"] == 1
    assert rec["waiter"] != 0  # rank 0 arrived late at everyone else
    b.close()


def _small_case(rr):
    R, count = 8, 8 * 20000 + 3
    x = workloads.generate(R, count, "fp32", "uniform_pm1", 31)
    return R, count, x, oracle_expect(x, "sum")


@pytest.mark.parametrize("sync", ["p2p", "barrier"])
@pytest.mark.parametrize("inject,waiter", [("extra", 0), ("drop", 1)])
def test_ring_timeout_then_recovery(rr, sync, inject, waiter):
    """A forced hand-off failure is reported with the missing count, later calls
    return at once while it is recorded, and clearing it restores normal work."""
    log(f"case ring timeout sync={sync} inject={inject}")
    R, count, x, expect = _small_case(rr)
    flag = rr.INJECT_EXTRA_EXPECTED if inject == "extra" else rr.INJECT_DROP_ARRIVAL
    slabs = to_slabs(rr, x, "fp32")
    rr.allreduce_ring(slabs.ranks, "sum", 4, sync=sync, inject=flag, timeout_ns=SHORT)
    torch.cuda.synchronize()
    # sticky: a second call does nothing while the failure is recorded
    before = slabs.storage.clone()
    rr.allreduce_ring(slabs.ranks, "sum", 4, sync=sync)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int32), slabs.storage.view(torch.int32))
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT
    assert rec["expected"] - rec["observed"] == 1
    if sync == "p2p":
        # the signal count is anonymous, so the predecessor's later arrivals stand in
        # for the missing one and the shortfall shows at the lane's last hand-off
        assert rec["ctx"] == 0 and rec["waiter"] == waiter and rec["hop"] == 2 * (R - 1)
    # recovered
    slabs = to_slabs(rr, x, "fp32")
    rr.allreduce_ring(slabs.ranks, "sum", 4, sync=sync)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert_matches_oracle([to_host(t, "fp32") for t in slabs.ranks], expect, "fp32", "recovered")


def test_check_kernel_error_raises(rr):
    R, count, x, expect = _small_case(rr)
    slabs = to_slabs(rr, x, "fp32")
    rr.allreduce_ring(slabs.ranks, "sum", 2, sync="p2p", inject=rr.INJECT_EXTRA_EXPECTED,
                      timeout_ns=SHORT)
    with pytest.raises(rr.RRError) as e:
        rr.check_kernel_error()
    assert "1 arrival(s) missing" in str(e.value)


def test_plan_of_the_benchmark_workload(rr):
    w = workloads.R8_FP32_64MIB
    p = rr.plan(w.R, w.count, w.dtype, w.nslices)
    assert p["sync"] == "p2p" and p["launches"] == 1
    assert p["grid"] <= p["resident_max"]
    assert p["chunk_len"] == w.count // w.R
    assert p["hbm_bytes"] == 5 * (w.R - 1) * w.count * 4
    p = rr.plan(64, 8 * 1024 * 1024, "fp32", 8, sync="barrier")
    assert p["sync"] == "barrier"
    cols = 8 * p["team"] // (p["depth"] * p["rounds"])
    assert p["grid"] == 64 * (-(-cols // 8) * 8)
    # too many lanes for one resident grid: auto falls back to one launch per hop
    p = rr.plan(64, 1 << 24, "fp32", 1024)
    assert p["sync"] == "launch" and p["launches"] == 126
    with pytest.raises(rr.RRError):
        rr.plan(64, 1 << 24, "fp32", 1024, sync="p2p")
