"""Pins of the oracle's staged loop and of the standalone ReduceScatter and
AllGather (no GPU).

* The primitive sequence of each rank is Table V as the loosp.cn post lists it
  (section 8; tests/golden/table_v_k4.txt for k = 4) and the general rule of
  section 10 (2k-1 steps).
* The chunk each rank receives at step k is the one the worked 4-GPU example
  sends it at round k (sections 5-6; tests/golden/worked_example_r4.txt).
* Traffic: counting each primitive's operands gives (6R-4)N for the AllReduce
  (send 2, recvReduceSend 3, recvReduceCopySend 4, recvCopySend 3, recv 2
  chunk-sized accesses) and (3R-1) chunk accesses per chunk for the standalone
  collectives.
* Values: brute force with exact arithmetic (oracle/brute.py), closed forms of
  tracer inputs, and the plain definition of a gather.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import brute
import workloads
from tests.test_oracle_pins import _parse_worked_example

RAW = {"int32": None, "fp32": np.uint32, "bf16": np.uint16, "fp16": np.uint16}
DIST = {"int32": "int_pm1000", "fp32": "uniform_pm1", "bf16": "normal", "fp16": "normal"}


def _bits(a, dtype):
    if dtype == "int32":
        return a.astype(np.int64)
    return a.view(RAW[dtype]).astype(np.int64)


def _table_v(R):
    return (["send"] + ["recvReduceSend"] * (R - 2) + ["recvReduceCopySend"] +
            ["recvCopySend"] * (R - 2) + ["recv"])


def test_staged_primitives_table_v_k4(golden_dir):
    with open(os.path.join(golden_dir, "table_v_k4.txt"), encoding="utf-8") as f:
        rows = [line.split() for line in f if line.strip() and not line.startswith("#")]
    want = [name for _, name in rows]
    x = workloads.generate(4, 64, "int32", "int_pm1000", 1)
    _, steps = oracle.staged_allreduce(x, log=True)
    for r in range(4):
        assert [s.prim for s in steps if s.rank == r] == want


@pytest.mark.parametrize("R", [2, 3, 5, 8, 16])
def test_staged_primitives_general(R):
    x = workloads.generate(R, 8 * R, "fp32", "uniform_pm1", 2)
    _, steps = oracle.staged_allreduce(x, log=True)
    for r in range(R):
        seq = [s.prim for s in steps if s.rank == r]
        assert seq == _table_v(R) and len(seq) == 2 * R - 1


def test_staged_chunks_follow_the_worked_example(golden_dir):
    rs, own, ag, final = _parse_worked_example(os.path.join(golden_dir, "worked_example_r4.txt"))
    x = workloads.generate(4, 64, "int32", "int_pm1000", 1)
    _, steps = oracle.staged_allreduce(x, log=True)
    by = {(s.step, s.rank): s.chunk for s in steps}
    for rnd, src, dst, chunk, _ in rs:       # ReduceScatter round k: dst receives at step k
        assert by[(rnd, dst)] == chunk
        assert by[(rnd - 1, src)] == chunk   # ... and src handled it the step before
    for rnd, src, dst, chunk in ag:
        if chunk is not None:
            assert by[(3 + rnd, dst)] == chunk
    for r, c in own.items():                 # the recvReduceCopySend step finishes the owned chunk
        assert by[(3, r)] == c


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16", "fp16"])
@pytest.mark.parametrize("R,count", [(2, 37), (3, 40), (5, 37 * 5 + 3), (8, 8 * 16 * 2 + 9)])
def test_staged_traffic(dtype, R, count):
    x = workloads.generate(R, count, dtype, DIST[dtype], 3)
    _, steps = oracle.staged_allreduce(x, log=True)
    N = count * workloads.ELEM_BYTES[dtype]
    assert sum(s.bytes_read + s.bytes_written for s in steps) == (6 * R - 4) * N


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16", "fp16"])
@pytest.mark.parametrize("op", ["sum", "max", "min", "prod"])
@pytest.mark.parametrize("R,count", [(2, 9), (4, 64), (5, 37), (8, 70)])
def test_staged_allreduce_brute_force(dtype, op, R, count):
    dist = "unit_jitter" if op == "prod" else DIST[dtype]
    x = workloads.generate(R, count, dtype, dist, 13 + R)
    keep = [a.copy() for a in x]
    y, _ = oracle.staged_allreduce(x, op)
    for a, b in zip(x, keep):  # out of place: the inputs are untouched
        assert np.array_equal(_bits(a, dtype), _bits(b, dtype))
    bounds = oracle.chunk_bounds(count, R, dtype)
    for i in range(count):
        c = int(np.searchsorted(bounds, i, side="right") - 1)
        vals = [int(x[r][i]) if dtype == "int32" else int(x[r].view(RAW[dtype])[i])
                for r in range(R)]
        want = brute.allreduce_element(vals, c, dtype, op)
        for r in range(R):
            assert int(_bits(y[r], dtype)[i]) == want


def test_staged_in_place():
    """recv == send: each rank reads a chunk of its input before writing it."""
    for dtype in ("fp32", "bf16"):
        x = workloads.generate(6, 6 * 8 * 3 + 5, dtype, DIST[dtype], 8)
        want, _ = oracle.staged_allreduce([a.copy() for a in x], "sum")
        buf = [a.copy() for a in x]
        oracle.staged_allreduce(buf, "sum", recv=buf)
        for a, b in zip(buf, want):
            assert np.array_equal(_bits(a, dtype), _bits(b, dtype))


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16", "fp16"])
@pytest.mark.parametrize("op", ["sum", "max", "min", "prod"])
@pytest.mark.parametrize("R,n", [(2, 5), (3, 7), (5, 4), (8, 9)])
def test_reduce_scatter_nccl_brute_force(dtype, op, R, n):
    """Rank r ends with block r, folded around the ring starting at rank r+1."""
    dist = "unit_jitter" if op == "prod" else DIST[dtype]
    x = workloads.generate(R, R * n, dtype, dist, 17 + R)
    y, steps = oracle.reduce_scatter_nccl(x, op, log=True)
    for r in range(R):
        for j in range(n):
            i = r * n + j
            vals = [int(x[q][i]) if dtype == "int32" else int(x[q].view(RAW[dtype])[i])
                    for q in range(R)]
            assert int(_bits(y[r], dtype)[j]) == brute.allreduce_element(vals, (r + 1) % R, dtype, op)
    es = workloads.ELEM_BYTES[dtype]
    assert sum(s.bytes_read + s.bytes_written for s in steps) == (3 * R - 1) * R * n * es
    for r in range(R):
        assert [s.prim for s in steps if s.rank == r] == \
            ["send"] + ["recvReduceSend"] * (R - 2) + ["recvReduceCopy"]


def test_reduce_scatter_nccl_tracers():
    R, n = 8, 13
    x = workloads.generate(R, R * n, "int32", "onehot", 0)
    y, _ = oracle.reduce_scatter_nccl(x, "sum")
    assert all(np.all(v == (1 << R) - 1) for v in y)
    x = workloads.generate(R, R * n, "int32", "rank_index", 0)
    y, _ = oracle.reduce_scatter_nccl(x, "sum")
    for r in range(R):   # sum over ranks q of q*1000 + i, i in block r
        i = np.arange(r * n, (r + 1) * n)
        assert np.array_equal(y[r], (sum(q * 1000 for q in range(R)) + R * i).astype(np.int32))


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16", "fp16"])
@pytest.mark.parametrize("R,n", [(2, 3), (5, 17), (8, 8)])
def test_all_gather_nccl_is_the_gather(dtype, R, n):
    x = workloads.generate(R, n, dtype, "bits", 23)
    y, steps = oracle.all_gather_nccl(x, log=True)
    want = np.concatenate([_bits(a, dtype) for a in x])
    for r in range(R):
        assert np.array_equal(_bits(y[r], dtype), want)
    es = workloads.ELEM_BYTES[dtype]
    assert sum(s.bytes_read + s.bytes_written for s in steps) == (3 * R - 1) * R * n * es
    for r in range(R):
        assert [s.prim for s in steps if s.rank == r] == \
            ["copySend"] + ["recvCopySend"] * (R - 2) + ["recv"]


@pytest.mark.parametrize("op", ["sum", "max", "min", "prod"])
def test_reduce_scatter_then_all_gather_nccl_is_allreduce_int32(op):
    """Integer reductions do not depend on the fold order, so the standalone
    pair equals the AllReduce of the same blocks."""
    R, n = 6, 11
    x = workloads.generate(R, R * n, "int32", "unit_jitter" if op == "prod" else "int_pm1000", 4)
    y, _ = oracle.reduce_scatter_nccl(x, op)
    z, _ = oracle.all_gather_nccl(y)
    ref = [a.copy() for a in x]
    oracle.allreduce(ref, op)
    for r in range(R):
        assert np.array_equal(z[r], ref[r])


def test_single_rank_is_a_copy():
    for dtype in ("fp32", "fp16"):
        x = workloads.generate(1, 10, dtype, "bits", 1)
        y, _ = oracle.staged_allreduce(x)
        assert np.array_equal(_bits(y[0], dtype), _bits(x[0], dtype))
        y, _ = oracle.reduce_scatter_nccl(x)
        assert np.array_equal(_bits(y[0], dtype), _bits(x[0], dtype))
        y, _ = oracle.all_gather_nccl(x)
        assert np.array_equal(_bits(y[0], dtype), _bits(x[0], dtype))


# ---------------------------------------------------------------- AlltoAll

@pytest.mark.parametrize("R,n", [(1, 5), (2, 3), (4, 16), (8, 37), (16, 9)])
def test_alltoall_pattern_of_the_gin_sample(R, n):
    """The GIN article's AlltoAll sample fills rank r's block for rank d with
    r*1000 + d*100 + i and checks that rank d receives, at block r, exactly
    that: the same pattern here (int32), so each block's source and place are
    both visible."""
    i = np.arange(n, dtype=np.int64)
    send = [np.concatenate([r * 1000 + d * 100 + i for d in range(R)]).astype(np.int32)
            for r in range(R)]
    recv = oracle.alltoall(send)
    for d in range(R):
        for r in range(R):
            assert np.array_equal(recv[d][r * n:(r + 1) * n], (r * 1000 + d * 100 + i).astype(np.int32))


def test_alltoall_is_a_byte_copy():
    R, n = 5, 33
    x = workloads.generate(R, R * n, "fp16", "bits", 3)   # NaN payloads included
    y = oracle.alltoall(x)
    z = oracle.alltoall(y)                                  # the exchange is its own inverse
    for a, b in zip(x, z):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
