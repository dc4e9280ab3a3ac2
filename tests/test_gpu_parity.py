"""GPU parity: the HIP ring kernels against the CPU oracle, element by element.

Every test compares every element of every rank with the oracle: small and
multi-tile sizes with guard bands checked too, the full-size workloads (up to
16 ranks x 1 GiB) one piece of each rank buffer at a time, plus sampled
positions and boundaries the oracle computes one by one and, for floating-point
SUM, the error bound against the order-free fp64 sum.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import (assert_full_matches, assert_matches_oracle, bits_equal, guards_intact,
                            log, oracle_at, oracle_expect, sample_positions, to_host, to_slabs)

pytestmark = pytest.mark.gpu

DIST = {"int32": "int_pm1000", "fp32": "uniform_pm1", "bf16": "normal"}


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_allreduce_amd
    ring_allreduce_amd.init()
    return ring_allreduce_amd


def run_case(rr, x, dtype, op, nslices, phase="allreduce", **opts):
    R, count = len(x), x[0].size
    slabs = to_slabs(rr, x, dtype)
    if phase == "allreduce":
        rr.allreduce_ring(slabs.ranks, op, nslices, **opts)
    elif phase == "reduce_scatter":
        rr.reduce_scatter_ring(slabs.ranks, op, nslices, **opts)
    else:
        rr.all_gather_ring(slabs.ranks, nslices, **opts)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert guards_intact(slabs, dtype, count), "a kernel wrote outside the rank buffers"
    return [to_host(t, dtype) for t in slabs.ranks]


# ----------------------------------------------------------- worked example

@pytest.mark.parametrize("sync", ["auto", "p2p", "barrier", "launch"])
def test_worked_example(rr, sync):
    w = workloads.WORKED_EXAMPLE
    log(f"case worked_example sync={sync}")
    x = workloads.inputs(w)
    got = run_case(rr, x, w.dtype, w.op, w.nslices, sync=sync)
    assert_matches_oracle(got, oracle_expect(x, w.op), w.dtype, "worked example")


# ------------------------------------------------------------ small, ragged

SMALL = [
    # R, count, nslices, team
    (2, 37, 1, 1), (3, 1000, 2, 1), (4, 4 * 4 * 7 + 3, 3, 2), (5, 12345, 4, 3),
    (8, 8 * 1024 + 5, 4, 2), (16, 16 * 8 * 33 + 7, 5, 1), (7, 6, 1, 1), (13, 9999, 16, 2),
]


@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("int32", "max"), ("fp32", "sum"),
                                      ("fp32", "max"), ("bf16", "sum"), ("bf16", "max")])
@pytest.mark.parametrize("R,count,nslices,team", SMALL)
@pytest.mark.parametrize("sync", ["p2p", "barrier", "launch"])
def test_small_ragged(rr, dtype, op, R, count, nslices, team, sync):
    log(f"case small {dtype} {op} R={R} count={count} ns={nslices} team={team} sync={sync}")
    x = workloads.generate(R, count, dtype, DIST[dtype], R * 31 + count % 97)
    got = run_case(rr, x, dtype, op, nslices, sync=sync, team=team)
    assert_matches_oracle(got, oracle_expect(x, op), dtype, f"R={R} count={count}")


@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("fp32", "sum"), ("bf16", "max"),
                                      ("bf16", "sum")])
@pytest.mark.parametrize("R,count,nslices,team", SMALL)
@pytest.mark.parametrize("depth", [1, 2])
def test_waiter_signal_small_ragged(rr, dtype, op, R, count, nslices, team, depth):
    """A barrier per hop through one counting signal per (lane, rank) that the
    R-1 other ranks add to (RR_FLAG_WAITER_SIGNAL; the default is one signal per
    lane): the same bits as the oracle."""
    if (nslices * team) % depth:
        pytest.skip("depth must divide the lanes")
    log(f"case waiter signal {dtype} {op} R={R} count={count} ns={nslices} team={team} "
        f"depth={depth}")
    x = workloads.generate(R, count, dtype, DIST[dtype], R * 37 + count % 89)
    got = run_case(rr, x, dtype, op, nslices, sync="barrier", team=team, depth=depth,
                   flags=rr.FLAG_WAITER_SIGNAL)
    assert_matches_oracle(got, oracle_expect(x, op), dtype, f"waiter R={R} count={count}")


# ------------------------------------- load policy (non-temporal incoming loads)

@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("fp32", "sum"), ("bf16", "max")])
@pytest.mark.parametrize("R,count,nslices,team", [SMALL[0], SMALL[3], SMALL[5], SMALL[7]])
@pytest.mark.parametrize("sync", ["p2p", "barrier", "launch"])
def test_stream_loads_small_ragged(rr, dtype, op, R, count, nslices, team, sync):
    """Small buffers take cached loads by default; forcing the non-temporal hint
    runs the other instantiation of every hop over the same ragged cases."""
    log(f"case stream loads {dtype} {op} R={R} count={count} ns={nslices} team={team} sync={sync}")
    x = workloads.generate(R, count, dtype, DIST[dtype], R * 31 + count % 97)
    want = oracle_expect(x, op)
    for opts in (dict(loads="stream"), dict(loads="stream", fused=True)):
        got = run_case(rr, x, dtype, op, nslices, sync=sync, team=team, **opts)
        assert_matches_oracle(got, want, dtype, f"R={R} count={count} {opts}")


@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("fp32", "sum"), ("bf16", "max")])
@pytest.mark.parametrize("R,count,nslices,team", [SMALL[0], SMALL[3], SMALL[5], SMALL[7]])
@pytest.mark.parametrize("sync", ["p2p", "barrier", "launch"])
def test_alternate_small_ragged(rr, dtype, op, R, count, nslices, team, sync):
    """Small buffers run every hop ascending by default; forcing the alternating
    direction (even hops top down) runs the other instantiation of every hop,
    ragged ends included, with and without the fused boundary."""
    log(f"case alternate {dtype} {op} R={R} count={count} ns={nslices} team={team} sync={sync}")
    x = workloads.generate(R, count, dtype, DIST[dtype], R * 43 + count % 83)
    want = oracle_expect(x, op)
    for opts in (dict(order="alternate"), dict(order="alternate", fused=True),
                 dict(order="alternate", loads="stream")):
        got = run_case(rr, x, dtype, op, nslices, sync=sync, team=team, **opts)
        assert_matches_oracle(got, want, dtype, f"R={R} count={count} {opts}")


def test_automatic_block_plan(rr):
    """Automatic workgroup size from the lane piece p, with the columns a
    512-thread plan would have: 128 if p <= 2 KiB, 256 if 16 KiB < p <= 32 KiB,
    128 if p <= 64 KiB on a long ring over buffers beyond the Infinity Cache,
    else 512; an explicit size is kept."""
    def pb(R, count, ns, sync, **kw):
        p = rr.plan(R, count, "fp32", ns, sync=sync, **kw)
        return p["block"], p["sub_len"] * 4, p
    for sync in ("p2p", "barrier"):
        b, piece, p = pb(64, 8 << 20, 8, sync)                  # 32 MiB per rank
        assert (b, piece) == ((128, 65536) if sync == "p2p" else (256, 32768))
        q = rr.plan(64, 8 << 20, "fp32", 8, sync=sync, block=512)
        assert (p["grid"], p["team"], p["depth"], p["rounds"]) == \
            (q["grid"], q["team"], q["depth"], q["rounds"])
    assert pb(16, 16 << 20, 4, "barrier")[:2] == (128, 65536)   # long ring, 1 GiB in all
    assert pb(16, 16 << 20, 4, "p2p")[:2] == (512, 131072)
    assert pb(8, 16 << 20, 4, "p2p")[:2] == (512, 65536)        # short ring
    assert pb(16, 4 << 20, 4, "barrier")[:2] == (256, 32768)    # 256 MiB in all
    assert pb(16, 1 << 10, 4, "p2p")[0] == 128                  # 4 KiB per rank
    assert pb(16, 1 << 18, 4, "p2p")[:2] == (512, 16384)        # 16 KiB: stays 512
    assert pb(64, 8 << 20, 8, "barrier", block=512)[0] == 512


def test_wide_barrier_block_plan(rr):
    """A barrier per hop on a long ring moving at least 1.5 GiB per hop (512 MiB per
    rank and more) runs one 1024-thread workgroup per CU, two lanes each, with the
    rounds of the 512-thread plan; predecessor hand-offs, shorter rings, smaller
    buffers and an explicit size keep the other rules."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for R, mib in ((16, 512), (16, 1024), (32, 512)):
        count = mib * (1 << 20) // 4
        p = rr.plan(R, count, "fp32", 4, sync="barrier")
        if cus % (8 * R):
            continue
        q = rr.plan(R, count, "fp32", 4, sync="p2p")
        assert (p["block"], p["grid"], p["depth"]) == (1024, cus, 2), p
        assert p["rounds"] == q["rounds"]
        assert q["block"] == 512
    assert rr.plan(16, 64 << 20, "fp32", 4, sync="barrier", block=512)["block"] == 512
    assert rr.plan(16, 32 << 20, "fp32", 4, sync="barrier")["block"] == 512    # 128 MiB
    assert rr.plan(16, 64 << 20, "bf16", 4, sync="barrier")["block"] == 512    # 128 MiB
    assert rr.plan(8, 256 << 20, "fp32", 4, sync="barrier")["block"] == 512    # short ring


def test_depth_and_rounds_plan(rr):
    """Automatic lanes per workgroup and rounds: predecessor hand-offs keep one
    lane and max(96 MiB, 12 MiB x R) of a hop in flight, except a long ring whose
    hop moves 384 MiB or more (two lanes, 384 MiB); a barrier per hop keeps two
    lanes and 48 MiB x R within [192, 384] MiB."""
    def dk(R, mib, sync, dtype="fp32", ns=4):
        p = rr.plan(R, mib * (1 << 20) // (4 if dtype == "fp32" else 2), dtype, ns, sync=sync)
        return p["depth"], p["rounds"]
    assert dk(8, 64, "p2p") == (1, 2)                       # 192 MiB per hop, 96 per round
    assert dk(8, 256, "p2p", "bf16", 8) == (1, 8)
    assert dk(64, 32, "p2p", ns=8) == (1, 1)                # 96 MiB per hop: not wide
    assert dk(16, 64, "p2p") == (1, 1)                      # 192 MiB per hop, 192 per round
    assert dk(16, 256, "p2p") == (2, 2)                     # wide: 768 MiB per hop
    assert dk(16, 1024, "p2p") == (2, 8)
    assert dk(64, 32, "barrier", ns=8) == (2, 1)
    assert dk(64, 256, "barrier") == (2, 2)                 # 384 MiB per round
    assert dk(16, 1024, "barrier") == (2, 8)
    assert dk(4, 256, "barrier") == (2, 4)                  # 192 MiB per round
    assert dk(8, 256, "barrier") == (2, 2)


def test_stream_loads_plan(rr):
    """Default: non-temporal once the R buffers exceed the 256 MB Infinity Cache."""
    assert rr.plan(8, 16 << 20, "fp32", 4)["stream_loads"] == 1        # 512 MiB
    assert rr.plan(16, 4 << 20, "fp32", 4)["stream_loads"] == 0        # 256 MiB: fits
    assert rr.plan(16, (4 << 20) + 4, "fp32", 4)["stream_loads"] == 1
    assert rr.plan(8, 16 << 20, "bf16", 4)["stream_loads"] == 0        # 256 MiB
    assert rr.plan(16, 1 << 10, "fp32", 4, loads="stream")["stream_loads"] == 1
    assert rr.plan(8, 16 << 20, "fp32", 4, loads="cached")["stream_loads"] == 0
    for phase in ("allreduce_staged", "reduce_scatter_blocks", "all_gather_blocks", "alltoall"):
        assert rr.plan(8, 16 << 20, "fp32", 1, phase=phase)["stream_loads"] == 0
    with pytest.raises(rr.RRError):
        rr.plan(8, 1024, "fp32", 1, flags=rr.FLAG_STREAM_LOADS | rr.FLAG_CACHED_LOADS)


def test_alternate_plan(rr):
    """Default: even hops top down once the R buffers exceed 128 MiB (half the
    Infinity Cache); the flags force either order; the staged kernel and the
    AlltoAll always run ascending."""
    assert rr.plan(8, 4 << 20, "fp32", 4)["alternate"] == 0            # 128 MiB
    assert rr.plan(8, (4 << 20) + 4, "fp32", 4)["alternate"] == 1
    assert rr.plan(16, 1 << 18, "fp32", 4)["alternate"] == 0           # 16 MiB
    assert rr.plan(16, 1 << 28, "fp32", 16, sync="barrier")["alternate"] == 1
    assert rr.plan(64, 8 << 20, "fp32", 8)["alternate"] == 1
    assert rr.plan(16, 1 << 10, "fp32", 4, order="alternate")["alternate"] == 1
    assert rr.plan(8, 16 << 20, "fp32", 4, order="ascending")["alternate"] == 0
    for phase in ("reduce_scatter", "all_gather"):
        assert rr.plan(8, 16 << 20, "fp32", 4, phase=phase)["alternate"] == 1
    for phase in ("allreduce_staged", "reduce_scatter_blocks", "all_gather_blocks", "alltoall"):
        assert rr.plan(8, 16 << 20, "fp32", 1, phase=phase)["alternate"] == 0
        assert rr.plan(8, 16 << 20, "fp32", 1, phase=phase, order="alternate")["alternate"] == 0
    with pytest.raises(rr.RRError):
        rr.plan(8, 1024, "fp32", 1, flags=rr.FLAG_ASCENDING | rr.FLAG_ALTERNATE)


# ----------------------------------------------- several tiles, default plan

MULTI = [(8, "fp32", "sum", (1 << 20) + 13, 4), (8, "bf16", "sum", (1 << 21) + 9, 8),
         (16, "fp32", "max", (1 << 20) + 3, 16), (4, "int32", "sum", 3 << 19, 2),
         (64, "fp32", "sum", 64 * 4096 + 5, 8)]


@pytest.mark.parametrize("R,dtype,op,count,nslices", MULTI)
@pytest.mark.parametrize("sync", ["auto", "barrier"])
def test_multi_tile(rr, R, dtype, op, count, nslices, sync):
    p = rr.plan(R, count, dtype, nslices, sync=sync)
    log(f"case multi R={R} {dtype} {op} count={count} ns={nslices} sync={sync} plan={p}")
    x = workloads.generate(R, count, dtype, DIST[dtype], 100 + R)
    got = run_case(rr, x, dtype, op, nslices, sync=sync)
    assert_matches_oracle(got, oracle_expect(x, op), dtype, f"multi R={R}")


@pytest.mark.parametrize("R,dtype,op,count,nslices", MULTI)
@pytest.mark.parametrize("sync", ["p2p", "barrier"])
def test_multi_tile_alternate(rr, R, dtype, op, count, nslices, sync):
    log(f"case multi alternate R={R} {dtype} {op} count={count} ns={nslices} sync={sync}")
    x = workloads.generate(R, count, dtype, DIST[dtype], 200 + R)
    want = oracle_expect(x, op)
    for order in ("alternate", "ascending"):
        got = run_case(rr, x, dtype, op, nslices, sync=sync, order=order)
        assert_matches_oracle(got, want, dtype, f"multi {order} R={R}")


@pytest.mark.parametrize("R,dtype,op,count,nslices", MULTI)
def test_multi_tile_stream_loads(rr, R, dtype, op, count, nslices):
    log(f"case multi stream R={R} {dtype} {op} count={count} ns={nslices}")
    x = workloads.generate(R, count, dtype, DIST[dtype], 100 + R)
    got = run_case(rr, x, dtype, op, nslices, sync="barrier", loads="stream")
    assert_matches_oracle(got, oracle_expect(x, op), dtype, f"multi stream R={R}")


@pytest.mark.parametrize("rounds,depth", [(1, 1), (2, 1), (4, 1), (8, 1), (1, 2), (2, 2),
                                          (1, 4), (2, 4), (1, 3)])
@pytest.mark.parametrize("sync", ["p2p", "barrier"])
def test_rounds_and_depth(rr, rounds, depth, sync):
    """Lane groups run one after another and lanes interleave hop by hop inside a
    workgroup: the same bits for every arrangement."""
    R, count, dtype, ns = 8, (1 << 20) + 13, "fp32", 4
    team = 8 if depth != 3 else 6
    p = rr.plan(R, count, dtype, ns, sync=sync, team=team, rounds=rounds, depth=depth)
    assert p["rounds"] == rounds and p["depth"] == depth
    cols = ns * team // (rounds * depth)
    assert p["grid"] == R * (-(-cols // 8) * 8)  # columns padded to a multiple of 8
    log(f"case rounds={rounds} depth={depth} sync={sync} plan={p}")
    x = workloads.generate(R, count, dtype, "uniform_pm1", 55)
    got = run_case(rr, x, dtype, "sum", ns, sync=sync, team=team, rounds=rounds, depth=depth)
    assert_matches_oracle(got, oracle_expect(x, "sum"), dtype, f"rounds {rounds} depth {depth}")


@pytest.mark.parametrize("dtype,op", [("bf16", "sum"), ("int32", "max")])
@pytest.mark.parametrize("depth", [2, 4])
def test_depth_small_ragged(rr, dtype, op, depth):
    R, count, ns = 5, 5 * 3000 + 7, 4
    x = workloads.generate(R, count, dtype, DIST[dtype], 66)
    for sync in ("p2p", "barrier"):
        log(f"case depth small {dtype} {op} depth={depth} sync={sync}")
        got = run_case(rr, x, dtype, op, ns, sync=sync, team=2, depth=depth)
        assert_matches_oracle(got, oracle_expect(x, op), dtype, f"depth {depth}")


# ------------------------------- fused boundary (recvReduceCopySend step)

FUSED_SMALL = [(2, 37, 1, 1), (3, 1000, 2, 1), (5, 12345, 4, 3), (8, 8 * 1024 + 5, 4, 2),
               (16, 16 * 8 * 33 + 7, 5, 1), (7, 6, 1, 1)]


@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("fp32", "sum"), ("fp32", "max"),
                                      ("bf16", "sum"), ("bf16", "max")])
@pytest.mark.parametrize("R,count,nslices,team", FUSED_SMALL)
@pytest.mark.parametrize("sync", ["p2p", "barrier", "launch"])
def test_fused_boundary_small(rr, dtype, op, R, count, nslices, team, sync):
    """The last ReduceScatter hop stores the finished chunk twice and the first
    AllGather hop moves nothing: the same bits as the plain ring."""
    log(f"case fused {dtype} {op} R={R} count={count} ns={nslices} team={team} sync={sync}")
    x = workloads.generate(R, count, dtype, DIST[dtype], R * 17 + count % 89)
    got = run_case(rr, x, dtype, op, nslices, sync=sync, team=team, fused=True)
    assert_matches_oracle(got, oracle_expect(x, op), dtype, f"fused R={R} count={count}")


@pytest.mark.parametrize("rounds,depth,sync", [(1, 1, "p2p"), (2, 2, "p2p"), (1, 4, "barrier"),
                                               (4, 1, "barrier"), (0, 0, "auto")])
def test_fused_boundary_multi_tile(rr, rounds, depth, sync):
    R, count, dtype, ns = 8, (1 << 20) + 13, "fp32", 4
    p = rr.plan(R, count, dtype, ns, sync=sync, rounds=rounds, depth=depth, fused=True)
    plain = rr.plan(R, count, dtype, ns, sync=sync, rounds=rounds, depth=depth)
    assert p["fused"] == 1 and plain["fused"] == 0
    assert p["hbm_bytes"] == plain["hbm_bytes"] - count * 4
    log(f"case fused multi rounds={rounds} depth={depth} sync={sync} plan={p}")
    x = workloads.generate(R, count, dtype, "uniform_pm1", 57)
    got = run_case(rr, x, dtype, "sum", ns, sync=sync, rounds=rounds, depth=depth, fused=True)
    assert_matches_oracle(got, oracle_expect(x, "sum"), dtype, "fused multi")


def test_fused_boundary_r64_and_phases(rr):
    R, count = 64, 64 * 4096 + 5
    x = workloads.generate(R, count, "bf16", "normal", 58)
    for sync in ("barrier", "p2p"):
        log(f"case fused R=64 sync={sync}")
        got = run_case(rr, x, "bf16", "sum", 8, sync=sync, fused=True)
        assert_matches_oracle(got, oracle_expect(x, "sum"), "bf16", f"fused R=64 {sync}")
    # the flag has no effect on a lone phase
    assert rr.plan(8, 1 << 16, "fp32", 2, phase="reduce_scatter", fused=True)["fused"] == 0
    x = workloads.generate(5, 5 * 999 + 1, "fp32", "uniform_pm1", 59)
    got = run_case(rr, x, "fp32", "sum", 2, phase="reduce_scatter", fused=True)
    assert_matches_oracle(got, oracle_expect(x, "sum", "reduce_scatter"), "fp32", "fused RS")


# ------------------------------------------------- the phases on their own

@pytest.mark.parametrize("dtype,op", [("fp32", "sum"), ("bf16", "sum"), ("int32", "max")])
@pytest.mark.parametrize("R", [2, 5, 8])
@pytest.mark.parametrize("sync", ["auto", "launch"])
def test_reduce_scatter_state(rr, dtype, op, R, sync):
    """Every chunk of every rank after ReduceScatter, partials included."""
    count = R * 3000 + 11
    log(f"case reduce_scatter {dtype} {op} R={R} sync={sync}")
    x = workloads.generate(R, count, dtype, DIST[dtype], 5 + R)
    got = run_case(rr, x, dtype, op, 3, phase="reduce_scatter", sync=sync)
    assert_matches_oracle(got, oracle_expect(x, op, "reduce_scatter"), dtype, "reduce_scatter")


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
@pytest.mark.parametrize("R", [2, 3, 8])
def test_all_gather_is_bitwise(rr, dtype, R):
    """Random bit patterns, NaN payloads included, are copied untouched."""
    count = R * 2048 + 5
    log(f"case all_gather bits {dtype} R={R}")
    x = workloads.generate(R, count, dtype, "bits", 77 + R)
    got = run_case(rr, x, dtype, "sum", 4, phase="all_gather")
    expect = oracle_expect(x, "sum", "all_gather")
    for r in range(R):
        assert np.array_equal(got[r].view(np.uint8), expect[r].view(np.uint8))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_reduce_scatter_then_all_gather(rr, dtype):
    R, count = 8, 8 * 10000 + 3
    log(f"case rs+ag {dtype}")
    x = workloads.generate(R, count, dtype, DIST[dtype], 3)
    slabs = to_slabs(rr, x, dtype)
    rr.reduce_scatter_ring(slabs.ranks, "sum", 4)
    rr.all_gather_ring(slabs.ranks, 4)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    got = [to_host(t, dtype) for t in slabs.ranks]
    assert_matches_oracle(got, oracle_expect(x, "sum"), dtype, "rs+ag")


# -------------------------------------------------------------- invariance

def test_invariance_across_slices_modes_teams(rr):
    """Slices, sync modes, teams and block sizes only schedule: bits never change."""
    R, count, dtype = 8, (1 << 18) + 17, "bf16"
    x = workloads.generate(R, count, dtype, "normal", 12)
    ref = None
    for nslices in (1, 2, 4, 8, 16):
        for sync in ("p2p", "barrier", "launch"):
            for team, block, depth in ((1, 256, 1), (4, 512, 2), (0, 1024, 0), (2, 128, 2)):
                log(f"case invariance ns={nslices} sync={sync} team={team} block={block}")
                got = run_case(rr, x, dtype, "sum", nslices, sync=sync, team=team, block=block,
                               depth=depth)
                if ref is None:
                    ref = got
                    assert_matches_oracle(got, oracle_expect(x, "sum"), dtype, "invariance")
                else:
                    for r in range(R):
                        assert np.array_equal(got[r], ref[r])


def test_repeat_runs_identical(rr):
    R, count, dtype = 16, 16 * 40000 + 1, "fp32"
    x = workloads.generate(R, count, dtype, "uniform_pm1", 4)
    expect = oracle_expect(x, "sum")
    slabs = to_slabs(rr, x, dtype)
    pristine = slabs.storage.clone()
    for k in range(10):
        log(f"case repeat {k}")
        slabs.storage.copy_(pristine)
        rr.allreduce_ring(slabs.ranks, "sum", 4)
        torch.cuda.synchronize()
        rr.check_kernel_error()
        got = [to_host(t, dtype) for t in slabs.ranks]
        assert_matches_oracle(got, expect, dtype, f"repeat {k}")


def test_no_xcd_map_and_cooperative(rr):
    R, count, dtype = 8, 8 * 50000 + 9, "fp32"
    x = workloads.generate(R, count, dtype, "uniform_pm1", 8)
    expect = oracle_expect(x, "sum")
    for flags in (rr.FLAG_NO_XCD_MAP, rr.FLAG_COOPERATIVE, 0):
        log(f"case flags={flags}")
        got = run_case(rr, x, dtype, "sum", 8, sync="p2p", flags=flags)
        assert_matches_oracle(got, expect, dtype, f"flags {flags}")


def test_separate_allocations(rr):
    """Rank buffers need not share one allocation."""
    R, count = 6, 6 * 7777 + 2
    x = workloads.generate(R, count, "fp32", "uniform_pm1", 2)
    ts = [torch.from_numpy(a).cuda() for a in x]
    log("case separate allocations")
    rr.allreduce_ring(ts, "sum", 2)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    expect = oracle_expect(x, "sum")
    assert_matches_oracle([t.cpu().numpy() for t in ts], expect, "fp32", "separate")


def test_edge_cases(rr):
    log("case edge: R=1, count=0, count<R")
    x = torch.randn(100, device="cuda")
    y = x.clone()
    rr.allreduce_ring([x], "sum", 1)
    torch.cuda.synchronize()
    assert torch.equal(x, y)
    e = [torch.empty(0, device="cuda") for _ in range(4)]
    rr.allreduce_ring(e, "sum", 1)
    xs = workloads.generate(8, 3, "int32", "int_pm1000", 1)
    got = run_case(rr, xs, "int32", "sum", 4)
    assert_matches_oracle(got, oracle_expect(xs, "sum"), "int32", "count<R")


def test_tracers(rr):
    R, count = 16, 16 * 4 * 9 + 1
    log("case tracers")
    x = workloads.generate(R, count, "int32", "onehot", 0)
    got = run_case(rr, x, "int32", "sum", 3)
    for g in got:
        assert np.all(g.view(np.int32) == (1 << R) - 1)
    x = workloads.generate(R, count, "int32", "rank", 0)
    got = run_case(rr, x, "int32", "max", 3)
    for g in got:
        assert np.all(g.view(np.int32) == R - 1)


def test_rolling_counters_near_wrap(rr):
    """Signals and shadows preset just below 2^64 must keep working past the wrap."""
    R, count = 8, 8 * 20000 + 3
    x = workloads.generate(R, count, "fp32", "uniform_pm1", 9)
    expect = oracle_expect(x, "sum")
    rr.workspace_preset((1 << 64) - 3)
    for sync, flags in (("p2p", 0), ("barrier", 0), ("barrier", rr.FLAG_WAITER_SIGNAL)):
        log(f"case wrap sync={sync} flags={flags}")
        got = run_case(rr, x, "fp32", "sum", 4, sync=sync, flags=flags)
        assert_matches_oracle(got, expect, "fp32", f"wrap {sync} {flags}")
    rr.workspace_preset(0)
    torch.cuda.synchronize()


def _hip():
    import ctypes
    # the soname the library links against: the HIP runtime already loaded
    lib = ctypes.CDLL("libamdhip64.so.7")
    lib.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    lib.hipFree.argtypes = [ctypes.c_void_p]
    lib.hipMemGetAddressRange.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    return lib


def test_invalid_device_pointers_rejected(rr):
    """A host pointer, or a buffer running past the end of its own allocation,
    never reaches a kernel: the call returns RR_ERR_INVALID.  The second buffer
    comes from a hipMalloc of its own (2 MiB, not from torch's caching
    allocator), whose extent the runtime is first asked for: the test goes on
    only if that extent is exactly what was allocated, so the library's check
    is the only thing between the call and a stray store."""
    import ctypes
    a = torch.zeros(1024, device="cuda")
    b = torch.zeros(1024, device="cuda")
    host = np.zeros(1024, dtype=np.float32)
    st = rr.allreduce_ring_ptrs([a.data_ptr(), host.ctypes.data], 1024, "fp32")
    assert st == rr.RR_ERR_INVALID
    hip = _hip()
    nbytes = 2 << 20
    p = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(p), nbytes) == 0
    try:
        tail = p.value + nbytes - 256 * 4        # 256 floats left in the allocation
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size),
                                         ctypes.c_void_p(tail)) == 0
        if base.value != p.value or size.value != nbytes:
            pytest.skip(f"the runtime reports an extent of {size.value} bytes for a "
                        f"{nbytes}-byte allocation")
        for count in (257, 1024):
            st = rr.allreduce_ring_ptrs([a.data_ptr(), b.data_ptr(), tail], count, "fp32")
            assert st == rr.RR_ERR_INVALID, count
        # exactly the bytes left: accepted (and run) -- the check is not too strict
        st = rr.allreduce_ring_ptrs([a.data_ptr(), b.data_ptr(), tail], 256, "fp32")
        assert st == rr.RR_OK
        torch.cuda.synchronize()
        rr.check_kernel_error()
    finally:
        torch.cuda.synchronize()
        assert hip.hipFree(p) == 0


# -------------------------------------------------------- full-size workloads

def _full_size(rr, w, n_random, opts=None):
    """The workload at its full size: every element of every rank against the
    oracle run on the same inputs (the oracle works in place on the host copy;
    the device output is read back one piece at a time), plus, on the original
    inputs, sampled positions and every chunk / slice / team boundary through
    the oracle one by one and, for floating-point SUM, the error bound against
    the order-free fp64 sum."""
    opts = opts or {}
    p = rr.plan(w.R, w.count, w.dtype, w.nslices, sync=w.sync, **opts)
    log(f"case full {w.name} R={w.R} {w.dtype} {w.op} count={w.count} ns={w.nslices} "
        f"sync={w.sync} plan={p}")
    x = workloads.inputs(w)
    slabs = to_slabs(rr, x, w.dtype, guard=True)
    rr.allreduce_ring(slabs.ranks, w.op, w.nslices, sync=w.sync, **opts)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert guards_intact(slabs, w.dtype, w.count)
    # sampled positions (boundaries included) through the oracle one by one
    pos = sample_positions(w.count, w.R, w.dtype, w.nslices, p, n_random, w.seed)
    idx = torch.from_numpy(pos).cuda()
    got = np.stack([to_host(t.index_select(0, idx), w.dtype) for t in slabs.ranks], axis=1)
    want = oracle_at(x, pos, w.dtype, w.op)
    eq = bits_equal(got, want.view(got.dtype), w.dtype)
    assert eq.all(), f"{np.count_nonzero(~eq)} of {eq.size} sampled results differ"
    # property: within the error bound of the order-free fp64 sum (floating point SUM)
    if w.op == "sum" and w.dtype != "int32":
        sub = [a[pos] for a in x]
        d, mag = oracle.direct_sum_f64(sub)
        y = got[:, 0]
        yv = (y.astype(np.uint32) << 16).view(np.float32) if w.dtype == "bf16" else y.view(np.float32)
        u = 2.0 ** -24 if w.dtype == "fp32" else 2.0 ** -8
        gamma = (w.R - 1) * u / (1 - (w.R - 1) * u)
        err = np.abs(yv.astype(np.float64) - d)
        assert np.all(err <= gamma * mag * (1 + 1e-12))
        if w.dtype == "fp32":
            assert np.all(err <= 1e-5 * mag)
        else:
            assert np.linalg.norm(yv - d) <= 1e-2 * np.linalg.norm(d)
    # every element of every rank
    oracle.allreduce(x, w.op)
    assert_full_matches(slabs.ranks, x, w.dtype, w.name)
    del slabs, x
    torch.cuda.empty_cache()


def test_full_r8_fp32_64MiB(rr):
    _full_size(rr, workloads.R8_FP32_64MIB, 20000)


@pytest.mark.parametrize("w", [workloads.R16_FP32_1GIB, workloads.R8_FP32_64MIB,
                               workloads.R8_BF16_256MIB, workloads.R64_FP32_32MIB],
                         ids=lambda w: w.name)
def test_full_size_in_the_bench_layout(rr, w):
    """The timed configurations themselves: one tensor per rank from bench.py's
    own buffer helper and the call bench.py times (same options), twice, each
    from the restored inputs as bench.py times them; both outputs compared with
    the oracle, every element of every rank."""
    import bench
    opts = dict(sync=w.sync, team=0, block=0, flags=0)
    p = rr.plan(w.R, w.count, w.dtype, w.nslices, **opts)
    log(f"case bench layout {w.name} plan={p}")
    x = workloads.inputs(w)
    tdt, raw_t, raw_np = ((torch.bfloat16, torch.int16, np.int16) if w.dtype == "bf16"
                          else (torch.float32, torch.int32, np.int32))
    ranks, snapshot = bench.rank_buffers(rr, torch, w.R, w.count, tdt, "separate")
    for r in range(w.R):
        ranks[r].view(raw_t).copy_(torch.from_numpy(x[r].view(raw_np)))
    restore = snapshot()
    oracle.allreduce(x, w.op)  # x now holds the expected output
    for call in range(2):
        restore()
        rr.allreduce_ring(ranks, w.op, w.nslices, **opts)
        torch.cuda.synchronize()
        rr.check_kernel_error()
        assert_full_matches(ranks, x, w.dtype, f"{w.name} call {call}")
    del ranks, restore, x
    torch.cuda.empty_cache()


def test_full_r8_bf16_256MiB(rr):
    _full_size(rr, workloads.R8_BF16_256MIB, 20000)


def test_full_r64_fp32_32MiB(rr):
    _full_size(rr, workloads.R64_FP32_32MIB, 3000)


@pytest.mark.parametrize("w", [workloads.R8_FP32_64MIB, workloads.R64_FP32_32MIB],
                         ids=lambda w: w.name)
def test_full_fused_boundary(rr, w):
    _full_size(rr, w, 5000, dict(fused=True))


@pytest.mark.parametrize("w", [workloads.R64_FP32_32MIB, workloads.r16_sweep(8, "sum", 16)],
                         ids=lambda w: w.name)
def test_full_waiter_signal(rr, w):
    """The barrier workloads with one counting signal per (lane, rank)."""
    _full_size(rr, w.with_(sync="barrier"), 4000, dict(flags=rr.FLAG_WAITER_SIGNAL))


def test_full_cached_loads(rr):
    """The default workload with the hint forced off (its default is on)."""
    _full_size(rr, workloads.R8_FP32_64MIB, 5000, dict(loads="cached"))


def test_full_stream_loads_in_cache(rr):
    """16 ranks x 16 MiB fit the Infinity Cache (default off); forced on."""
    _full_size(rr, workloads.r16_sweep(6, "sum", 4), 5000, dict(loads="stream"))


@pytest.mark.parametrize("k", range(0, 9))
def test_full_r16_sweep(rr, k):
    for op, ns in (("sum", 16), ("max", 1 + (k % 4) * 5)):
        _full_size(rr, workloads.r16_sweep(k, op, ns), 4000)


def test_full_r16_p2p_two_lanes(rr):
    """Predecessor hand-offs with two lanes per workgroup (the automatic plan of
    a long ring with a wide hop): 16 ranks x 256 MiB."""
    w = workloads.r16_sweep(8, "sum", 4).with_(sync="p2p")
    p = rr.plan(w.R, w.count, w.dtype, w.nslices, sync="p2p")
    assert p["depth"] == 2 and p["sync"] == "p2p"
    _full_size(rr, w, 4000)


def test_full_r16_1GiB(rr):
    """The largest point of the R=16 sweep: 1 GiB per rank, 16 GiB in all."""
    _full_size(rr, workloads.r16_sweep(9, "sum", 16), 3000)


def test_full_r16_1GiB_barrier(rr):
    """The same point with a barrier per hop: the wide-hop plan (one 1024-thread
    workgroup per CU, two lanes each)."""
    w = workloads.r16_sweep(9, "max", 4).with_(sync="barrier")
    p = rr.plan(w.R, w.count, w.dtype, w.nslices, sync="barrier")
    log(f"case full r16 1GiB barrier plan={p}")
    _full_size(rr, w, 3000)


def test_wide_barrier_plan_mid_size(rr):
    """The wide barrier plan's shape (1024 threads, one workgroup per CU, two lanes,
    several rounds) forced on 32 ranks x 4 MiB + a ragged tail, against the oracle."""
    R, count, ns, cols = 32, (1 << 20) + 4 * 32 * 7 + 3, 4, 8
    for op, dtype in (("sum", "fp32"), ("max", "bf16")):
        x = workloads.generate(R, count, dtype, DIST[dtype], 501)
        opts = dict(sync="barrier", block=1024, team=cols * 2 * 2 // ns, depth=2, rounds=2)
        p = rr.plan(R, count, dtype, ns, **opts)
        assert (p["block"], p["depth"], p["rounds"]) == (1024, 2, 2), p
        log(f"case wide barrier shape R={R} {dtype} {op} plan={p}")
        got = run_case(rr, x, dtype, op, ns, **opts)
        assert_matches_oracle(got, oracle_expect(x, op), dtype, f"wide barrier {dtype} {op}")


def test_pieces_longer_than_one_descriptor(rr):
    """A workgroup's range over 1 GiB is moved in parts (each buffer descriptor
    covers at most 1 GiB): R=2, 2 GiB per rank, one slice, one team member, in
    the ring and in the staged loop."""
    R, count = 2, (1 << 29) + 37          # fp32: 2 GiB + 148 B per rank
    w = workloads.Workload("r2_fp32_2GiB", R, "fp32", "sum", count, 1, 97, "uniform_pm1")
    p = rr.plan(R, count, "fp32", 1, team=1)
    assert p["sub_len"] * 4 > (1 << 30)
    log(f"case big pieces plan={p}")
    x = workloads.inputs(w)
    send = to_slabs(rr, x, "fp32", guard=True)
    recv = rr.allreduce_ring_staged(send.ranks, None, "sum", 1, team=1)
    rr.allreduce_ring(send.ranks, "sum", 1, team=1)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert guards_intact(send, "fp32", count)
    for r in range(R):
        assert torch.equal(send.ranks[r].view(torch.int32), recv[r].view(torch.int32))
    pos = sample_positions(count, R, "fp32", 1, p, 20000, 97)
    pos = np.unique(np.concatenate([pos, (1 << 28) - 2 + np.arange(4),   # around 1 GiB into chunk 0
                                    (p["chunk_len"] + (1 << 28)) - 2 + np.arange(4)]))
    pos = pos[pos < count]
    idx = torch.from_numpy(pos).cuda()
    got = np.stack([to_host(t.index_select(0, idx), "fp32") for t in send.ranks], axis=1)
    want = oracle_at(x, pos, "fp32", "sum")
    assert bits_equal(got, want.view(got.dtype), "fp32").all()
    # every element of both ranks, in place and staged
    oracle.allreduce(x, "sum")
    assert_full_matches(send.ranks, x, "fp32", "ring, 2 GiB per rank")
    assert_full_matches(recv, x, "fp32", "staged, 2 GiB per rank")


@pytest.mark.parametrize("sync,flags", [("p2p", 0), ("barrier", 0), ("barrier", "waiter")])
def test_hop_stamps(rr, sync, flags):
    """allreduce_ring_timed: the same bits as the oracle, and stamps that respect
    the hand-off order.  Per (lane, rank, hop): wait begins <= hop begins <= hop
    ends.  A hop begins only after the hop it waits for has begun: the
    predecessor's previous hop (P2P), every rank's previous hop (barrier)."""
    R, count, ns = 8, 8 * 4096 * 3 + 5, 3
    f = rr.FLAG_WAITER_SIGNAL if flags == "waiter" else 0
    log(f"case hop stamps sync={sync} flags={f}")
    x = workloads.generate(R, count, "fp32", "uniform_pm1", 61)
    slabs = to_slabs(rr, x, "fp32")
    stamps, khz = rr.allreduce_ring_timed(slabs.ranks, "sum", ns, sync=sync, flags=f)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert khz > 0
    assert guards_intact(slabs, "fp32", count)
    assert_matches_oracle([to_host(t, "fp32") for t in slabs.ranks], oracle_expect(x, "sum"),
                          "fp32", "timed call")
    st = stamps.cpu().numpy().astype(np.int64)            # (lanes, R, hops, 3)
    p = rr.plan(R, count, "fp32", ns, sync=sync)
    assert st.shape == (ns * p["team"], R, 2 * (R - 1), 3)
    assert (st > 0).all()
    assert (st[..., 0] <= st[..., 1]).all() and (st[..., 1] <= st[..., 2]).all()
    # the first hop does not wait: its first two stamps are two clock reads in a row
    assert ((st[:, :, 0, 1] - st[:, :, 0, 0]) * 1e6 / (khz * 1e3) < 5.0).all()
    begin = st[..., 1]
    for g in range(1, 2 * (R - 1)):
        if sync == "p2p":
            prev = np.roll(begin[:, :, g - 1], 1, axis=1)  # rank r-1's previous hop
        else:
            prev = begin[:, :, g - 1].max(axis=1, keepdims=True)
        assert (begin[:, :, g] >= prev).all(), g
