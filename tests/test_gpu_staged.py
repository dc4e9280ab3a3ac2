"""GPU parity of the staged, out-of-place loop (Table V of the loosp.cn post) and
of the standalone ReduceScatter and AllGather, against the CPU oracle, bit for
bit.  Send buffers must come back untouched and nothing may be written outside
the receive buffers (guard bands)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import (RAW_NP, assert_full_matches, assert_matches_oracle, bits_equal,
                            guards_intact, log, oracle_at, oracle_expect, sample_positions,
                            to_device, to_host, to_slabs)

pytestmark = pytest.mark.gpu

DIST = {"int32": "int_pm1000", "fp32": "uniform_pm1", "bf16": "normal", "fp16": "normal"}


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_allreduce_amd
    ring_allreduce_amd.init()
    return ring_allreduce_amd


def _dist(dtype, op):
    return "unit_jitter" if op == "prod" else DIST[dtype]


def _staged(rr, x, dtype, op, nslices, **opts):
    R, count = len(x), x[0].size
    send = to_slabs(rr, x, dtype)
    before = send.storage.clone()
    recv = to_slabs(rr, [np.zeros_like(a) for a in x], dtype)
    rr.allreduce_ring_staged(send.ranks, recv.ranks, op, nslices, **opts)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert torch.equal(send.storage.view(torch.int16), before.view(torch.int16)), "input changed"
    assert guards_intact(recv, dtype, count), "a kernel wrote outside the receive buffers"
    return [to_host(t, dtype) for t in recv.ranks]


SMALL = [(2, 37, 1), (3, 1000, 2), (4, 4 * 4 * 7 + 3, 3), (5, 12345, 4), (8, 8 * 1024 + 5, 4),
         (16, 16 * 8 * 33 + 7, 5), (7, 6, 1)]


@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("int32", "prod"), ("fp32", "sum"),
                                      ("fp32", "max"), ("bf16", "sum"), ("bf16", "min"),
                                      ("fp16", "sum"), ("fp16", "prod")])
@pytest.mark.parametrize("R,count,nslices", SMALL)
@pytest.mark.parametrize("sync", ["p2p", "launch"])
def test_staged_small_ragged(rr, dtype, op, R, count, nslices, sync):
    log(f"case staged {dtype} {op} R={R} count={count} ns={nslices} sync={sync}")
    x = workloads.generate(R, count, dtype, _dist(dtype, op), R * 13 + count % 83)
    got = _staged(rr, x, dtype, op, nslices, sync=sync)
    assert_matches_oracle(got, oracle_expect(x, op), dtype, f"staged R={R} count={count}")


def test_staged_equals_the_oracles_staged_loop(rr):
    R, count = 6, 6 * 1000 + 9
    x = workloads.generate(R, count, "bf16", "normal", 61)
    want, _ = oracle.staged_allreduce(x, "sum")
    got = _staged(rr, x, "bf16", "sum", 3)
    assert_matches_oracle(got, want, "bf16", "staged vs staged oracle")


@pytest.mark.parametrize("R,count,ns", [(8, (1 << 20) + 13, 4), (64, 64 * 4096 + 5, 8),
                                        (4, 3 << 19, 2)])
def test_staged_multi_tile_and_plan(rr, R, count, ns):
    p = rr.plan(R, count, "fp32", ns, phase="allreduce_staged")
    assert p["hbm_bytes"] == (6 * R - 4) * count * 4
    log(f"case staged multi R={R} count={count} plan={p}")
    x = workloads.generate(R, count, "fp32", "uniform_pm1", 62)
    got = _staged(rr, x, "fp32", "sum", ns)
    assert_matches_oracle(got, oracle_expect(x, "sum"), "fp32", f"staged multi R={R}")


def test_staged_in_place(rr):
    R, count = 5, 5 * 7777 + 3
    x = workloads.generate(R, count, "fp32", "uniform_pm1", 63)
    slabs = to_slabs(rr, x, "fp32")
    log("case staged in place")
    rr.allreduce_ring_staged(slabs.ranks, slabs.ranks, "sum", 4)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert guards_intact(slabs, "fp32", count)
    assert_matches_oracle([to_host(t, "fp32") for t in slabs.ranks], oracle_expect(x, "sum"),
                          "fp32", "staged in place")


def test_staged_repeat_and_team(rr):
    R, count = 8, 8 * 40000 + 11
    x = workloads.generate(R, count, "fp16", "normal", 64)
    want = oracle_expect(x, "sum")
    for opts in ({}, dict(team=1), dict(team=7), dict(team=3, sync="launch"), {}):
        log(f"case staged opts={opts}")
        got = _staged(rr, x, "fp16", "sum", 4, **opts)
        assert_matches_oracle(got, want, "fp16", f"staged {opts}")


@pytest.mark.parametrize("rounds,team", [(2, 4), (4, 4), (3, 3), (8, 2)])
def test_staged_rounds(rr, rounds, team):
    """Lane groups run one after another: the same bits for every grouping."""
    R, count, ns = 8, (1 << 20) + 13, 4
    p = rr.plan(R, count, "bf16", ns, phase="allreduce_staged", rounds=rounds, team=team)
    assert p["rounds"] == rounds and p["team"] == team
    log(f"case staged rounds={rounds} team={team} plan={p}")
    x = workloads.generate(R, count, "bf16", "normal", 65)
    got = _staged(rr, x, "bf16", "sum", ns, rounds=rounds, team=team)
    assert_matches_oracle(got, oracle_expect(x, "sum"), "bf16", f"staged rounds {rounds}")
    y = workloads.generate(R, R * 5001, "fp32", "uniform_pm1", 66)
    recv = rr.reduce_scatter(_blocks_send(y, "fp32"), None, "sum", ns, rounds=rounds, team=team)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    want, _ = oracle.reduce_scatter_nccl(y, "sum")
    assert_matches_oracle([to_host(t, "fp32") for t in recv], want, "fp32", "RS rounds")


def test_staged_single_rank_and_empty(rr):
    x = torch.randn(1000, device="cuda")
    y = rr.allreduce_ring_staged([x])[0]
    torch.cuda.synchronize()
    assert torch.equal(x, y)
    e = [torch.empty(0, device="cuda") for _ in range(3)]
    rr.allreduce_ring_staged(e, [torch.empty(0, device="cuda") for _ in range(3)])


# ------------------------------------------------- standalone collectives

def _blocks_send(x, dtype):
    return [to_device(a, dtype) for a in x]


@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("fp32", "sum"), ("fp32", "min"),
                                      ("bf16", "sum"), ("fp16", "prod"), ("int32", "max")])
@pytest.mark.parametrize("R,n", [(2, 37), (3, 64), (5, 1001), (8, 4096), (8, 4099), (16, 333)])
@pytest.mark.parametrize("sync", ["p2p", "launch"])
def test_reduce_scatter_blocks(rr, dtype, op, R, n, sync):
    log(f"case reduce_scatter {dtype} {op} R={R} n={n} sync={sync}")
    x = workloads.generate(R, R * n, dtype, _dist(dtype, op), 70 + R)
    send = _blocks_send(x, dtype)
    recv = rr.reduce_scatter(send, None, op, 2, sync=sync)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    want, _ = oracle.reduce_scatter_nccl(x, op)
    got = [to_host(t, dtype) for t in recv]
    assert_matches_oracle(got, want, dtype, f"reduce_scatter R={R} n={n}")
    for a, t in zip(x, send):
        assert np.array_equal(to_host(t, dtype), a.view(RAW_NP[dtype]))


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16", "fp16"])
@pytest.mark.parametrize("R,n", [(2, 5), (3, 64), (5, 1001), (8, 4096), (16, 333)])
@pytest.mark.parametrize("sync", ["p2p", "launch"])
def test_all_gather_blocks(rr, dtype, R, n, sync):
    log(f"case all_gather {dtype} R={R} n={n} sync={sync}")
    x = workloads.generate(R, n, dtype, "bits", 80 + R)
    recv = rr.all_gather(_blocks_send(x, dtype), None, 3, sync=sync)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    want = np.concatenate([a.view(RAW_NP[dtype]) for a in x])
    for t in recv:
        assert np.array_equal(to_host(t, dtype), want)


def test_standalone_plans_and_single_rank(rr):
    p = rr.plan(8, 4096, "fp32", 2, phase="reduce_scatter_blocks")
    assert p["hbm_bytes"] == (3 * 8 - 1) * 8 * 4096 * 4
    p = rr.plan(8, 4096, "bf16", 2, phase="all_gather_blocks")
    assert p["hbm_bytes"] == (3 * 8 - 1) * 8 * 4096 * 2
    x = torch.randn(64, device="cuda")
    assert torch.equal(rr.reduce_scatter([x])[0], x)
    assert torch.equal(rr.all_gather([x])[0], x)
    torch.cuda.synchronize()


def test_reduce_scatter_then_all_gather_int32(rr):
    """Integer reductions do not depend on the fold order: the standalone pair
    equals the in-place ring's AllReduce of the same buffers."""
    R, n = 8, 50001
    x = workloads.generate(R, R * n, "int32", "int_pm1000", 90)
    y = rr.reduce_scatter(_blocks_send(x, "int32"), None, "sum", 4)
    z = rr.all_gather(y, None, 4)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    want = oracle_expect(x, "sum")
    assert_matches_oracle([to_host(t, "int32") for t in z], want, "int32", "RS + AG")


def test_staged_timeout_and_recovery(rr):
    R, count = 8, 8 * 20000 + 3
    x = workloads.generate(R, count, "fp32", "uniform_pm1", 91)
    send = to_slabs(rr, x, "fp32")
    recv = to_slabs(rr, [np.zeros_like(a) for a in x], "fp32")
    log("case staged timeout")
    rr.allreduce_ring_staged(send.ranks, recv.ranks, "sum", 4, sync="p2p",
                             inject=rr.INJECT_DROP_ARRIVAL, timeout_ns=20_000_000)
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT and rec["expected"] - rec["observed"] >= 1
    got = _staged(rr, x, "fp32", "sum", 4)
    assert_matches_oracle(got, oracle_expect(x, "sum"), "fp32", "staged recovered")


# -------------------------------------------------------------- full size

def test_staged_full_r8_fp32_64MiB(rr):
    w = workloads.R8_FP32_64MIB
    p = rr.plan(w.R, w.count, w.dtype, w.nslices, phase="allreduce_staged")
    log(f"case staged full {w.name} plan={p}")
    x = workloads.inputs(w)
    send = to_slabs(rr, x, w.dtype, guard=True)
    recv = to_slabs(rr, [np.zeros_like(a) for a in x], w.dtype, guard=True)
    rr.allreduce_ring_staged(send.ranks, recv.ranks, w.op, w.nslices)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert guards_intact(recv, w.dtype, w.count)
    raw = [t.view(torch.int32) for t in recv.ranks]
    for r in range(1, w.R):
        assert torch.equal(raw[r], raw[0])
    # the same bits as the in-place ring
    rr.allreduce_ring(send.ranks, w.op, w.nslices)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert torch.equal(send.ranks[3].view(torch.int32), raw[3])
    pos = sample_positions(w.count, w.R, w.dtype, w.nslices, p, 20000, w.seed)
    idx = torch.from_numpy(pos).cuda()
    got = np.stack([to_host(t.index_select(0, idx), w.dtype) for t in recv.ranks], axis=1)
    want = oracle_at(x, pos, w.dtype, w.op)
    assert bits_equal(got, want.view(got.dtype), w.dtype).all()
    # every element of every rank
    expect, _ = oracle.staged_allreduce(x, w.op)
    assert_full_matches(recv.ranks, expect, w.dtype, "staged full")


def test_reduce_scatter_full_size_unaligned(rr):
    R, n = 8, (1 << 21) + 3   # blocks not a multiple of 16 bytes: the element path
    x = workloads.generate(R, R * n, "fp32", "uniform_pm1", 92)
    log("case reduce_scatter full unaligned")
    y = rr.reduce_scatter(_blocks_send(x, "fp32"), None, "sum", 4)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    want, _ = oracle.reduce_scatter_nccl(x, "sum")
    assert_matches_oracle([to_host(t, "fp32") for t in y], want, "fp32", "RS full")
