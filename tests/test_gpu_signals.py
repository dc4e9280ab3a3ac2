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


@pytest.mark.parametrize("R,nctx", [(2, 1), (8, 4), (64, 8)])
def test_shared_barrier_counts(rr, R, nctx):
    """One signal per context that every waiter adds 1 to: it advances by R per
    step, every waiter's shadow of it follows, and the per-waiter signals are
    untouched."""
    log(f"case shared barrier counts R={R} nctx={nctx}")
    b = rr.CountingBarrier(64, 8)
    b.run(R, 50, nctx, mode="shared")
    torch.cuda.synchronize()
    rr.check_kernel_error()
    for ctx in range(nctx):
        assert b.read(ctx, -1) == (50 * R, 50 * R)
        assert b.read(ctx, 0) == (0, 0)
    if nctx < 8:
        assert b.read(nctx, -1) == (0, 0)
    b.run(R, 7, nctx, mode="shared")
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert b.read(0, -1) == (57 * R, 57 * R)
    b.close()


def test_shared_barrier_timeout_and_drop(rr):
    """Shared layout: an expectation of R+1 per step, or a dropped arrival, times
    out with one arrival missing; after reading the record and a reset the
    barrier counts again."""
    log("case shared barrier timeout")
    b = rr.CountingBarrier(8, 2)
    b.run(8, 5, 2, expected=9, mode="shared", timeout_ns=SHORT)
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT and rec["expected"] - rec["observed"] == 1
    b.reset()
    b.run(8, 3, 1, mode="shared", inject=rr.INJECT_DROP_ARRIVAL, timeout_ns=SHORT)
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT and rec["expected"] - rec["observed"] == 1
    b.reset()
    b.run(8, 5, 2, mode="shared")
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert b.read(1, -1) == (40, 40)
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


# ------------------------------------------- per-peer slots vs counting signal

@pytest.mark.parametrize("R,nctx", [(2, 1), (8, 4), (64, 8)])
def test_per_peer_barrier_counts(rr, R, nctx):
    log(f"case per-peer counts R={R} nctx={nctx}")
    b = rr.CountingBarrier(64, 8)
    steps = 40
    b.run(R, steps, nctx, mode="per_peer")
    torch.cuda.synchronize()
    rr.check_kernel_error()
    for ctx in range(nctx):
        for q in (0, R // 2, R - 1):
            for p in {(q + 1) % R, (q + R - 1) % R}:
                if p != q:
                    assert b.read_peer(ctx, q, p) == (steps, steps)
            assert b.read(ctx, q) == (0, 0)  # the counting signals are not used
    b.run(R, 3, nctx, mode="per_peer")
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert b.read_peer(0, R - 1, 0) == (steps + 3, steps + 3)
    b.close()


def test_per_peer_barrier_wraps(rr):
    b = rr.CountingBarrier(8, 1)
    start = (1 << 64) - 2
    b.preset(start)
    b.run(8, 6, 1, mode="per_peer")
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert b.read_peer(0, 5, 2) == ((start + 6) % (1 << 64),) * 2
    b.close()


def test_per_peer_timeout_names_the_peer(rr):
    """A per-peer slot knows who is missing; the record names that peer."""
    log("case per-peer timeout")
    b = rr.CountingBarrier(8, 1)
    b.run(8, 3, 1, mode="per_peer", inject=rr.INJECT_DROP_ARRIVAL, timeout_ns=SHORT)
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT
    assert 0 <= rec["peer"] < 8 and rec["peer"] != rec["waiter"]
    value, _ = b.read_peer(rec["ctx"], rec["waiter"], rec["peer"])
    assert value == rec["observed"] < rec["expected"]
    # Rank 0 skipped its step-1 arrivals.  Its later arrivals still come from
    # rank 0, so each slot lets the others through steps 1 and 2 one arrival
    # late, and the shortfall shows at the last step, where the record names
    # rank 0 as the missing peer.
    assert rec["peer"] == 0 and rec["waiter"] != 0 and rec["hop"] == 3
    for q in range(1, 8):
        assert b.read_peer(0, q, 0)[0] == 2
    b.close()


@pytest.mark.parametrize("R", [3, 8, 64])
def test_deferred_arrival_counting_passes_on_a_stand_in(rr, R):
    """Waiter 0 holds back its step-1 and step-2 arrivals at waiter 1 until it
    has passed step 2.  The counting barrier completes anyway: another peer one
    step ahead fills waiter 1's step-1 count, which the audit witnesses record
    as an early pass."""
    log(f"case defer counting R={R}")
    b = rr.CountingBarrier(64, 1)
    steps = 6
    b.run(R, steps, 1, mode="barrier", inject=rr.INJECT_DEFER_ARRIVAL, flags=rr.FLAG_AUDIT)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert b.early_passes(0, 1) >= 1
    for q in range(R):
        assert b.read(0, q) == (steps * (R - 1),) * 2
    assert b.read_peer(0, 1, 0) == (steps, steps)  # every witness caught up by the end
    b.close()


@pytest.mark.parametrize("R,mode", [(3, "per_peer"), (8, "per_peer"), (2, "barrier")])
def test_deferred_arrival_blocks_identity_barriers(rr, R, mode):
    """Per-peer slots (and a counting barrier with a single peer) cannot pass
    without that arrival: the held-back arrival never comes, the waits time out,
    and the record names a waiter whose wait was truly unmet."""
    log(f"case defer blocks R={R} mode={mode}")
    b = rr.CountingBarrier(8, 1)
    b.run(R, 4, 1, mode=mode, inject=rr.INJECT_DEFER_ARRIVAL, timeout_ns=SHORT)
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT
    if mode == "per_peer":
        value, _ = b.read_peer(rec["ctx"], rec["waiter"], rec["peer"])
        assert value == rec["observed"] < rec["expected"]
        assert b.read_peer(0, 1, 0)[0] == 0
    else:
        assert rec["peer"] == -1  # a counting signal cannot name the peer
    b.close()


def test_audit_without_injection(rr):
    """Audited counting runs and per-peer runs keep every count exact; per-peer
    runs never count early passes."""
    R, steps = 16, 200
    b = rr.CountingBarrier(16, 2)
    b.run(R, steps, 2, mode="barrier", flags=rr.FLAG_AUDIT)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    for q in range(R):
        assert b.read(1, q) == (steps * (R - 1),) * 2
        assert b.read_peer(1, q, (q + 3) % R) == (steps, steps)
    early = sum(b.early_passes(c, q) for c in range(2) for q in range(R))
    log(f"audited counting barrier R={R}: {early} early passes in {2 * R * steps} waits")
    b.reset()
    b.run(R, steps, 2, mode="per_peer", flags=rr.FLAG_AUDIT)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert all(b.early_passes(c, q) == 0 for c in range(2) for q in range(R))
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


@pytest.mark.parametrize("mode", ["barrier", "shared", "per_peer", "p2p"])
@pytest.mark.parametrize("R,nctx", [(2, 1), (5, 3), (16, 2), (64, 8)])
def test_step_stamps_show_the_ordering(rr, mode, R, nctx):
    """In-kernel step times (one device-wide constant-rate clock): every waiter's
    stamps are non-decreasing, and no waiter leaves step k before the peers it
    waits for have left step k-1 (all other waiters of its context for the
    counting and per-peer barriers, the predecessor for p2p).  The stamp of step
    k-1 is taken before the peer's step-k arrival, which the waiter must see
    before taking its own stamp of step k, so the order is strict in time."""
    log(f"case stamps mode={mode} R={R} nctx={nctx}")
    b = rr.CountingBarrier(64, 8)
    nsteps = 200
    st, khz = b.run_timed(R, nsteps, nctx, mode=mode)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert khz > 0
    s = st.cpu().numpy()
    assert s.shape == (nctx, R, nsteps + 1)
    assert (s > 0).all()
    assert (np.diff(s, axis=2) >= 0).all()
    before, after = s[:, :, :-1], s[:, :, 1:]      # step k-1 and step k, k = 1..nsteps
    if mode == "p2p":
        pred = np.roll(before, 1, axis=1)            # waiter q's predecessor q-1
        assert (after >= pred).all()
    else:
        for q in range(R):
            others = np.delete(before, q, axis=1).max(axis=1)
            assert (after[:, q] >= others).all(), f"waiter {q} left a step early"
    # the untimed run counts the same as the timed one
    for c in range(nctx):
        for q in (range(R) if mode != "shared" else [-1]):
            v, sh = b.read(c, q)
            assert v == sh
    b.close()
