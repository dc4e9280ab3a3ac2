"""GPU parity of the in-place ring for fp16, for MIN and PROD, and for special
values in every type: the HIP kernels against the CPU oracle, element by element,
bit for bit."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import (assert_full_matches, assert_matches_oracle, guards_intact, log,
                            oracle_expect, to_host, to_slabs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_allreduce_amd
    ring_allreduce_amd.init()
    return ring_allreduce_amd


def _dist(dtype, op):
    if op == "prod":
        return "unit_jitter"
    return {"int32": "int_pm1000", "fp32": "uniform_pm1", "bf16": "normal", "fp16": "normal"}[dtype]


def _run(rr, x, dtype, op, nslices, **opts):
    slabs = to_slabs(rr, x, dtype)
    rr.allreduce_ring(slabs.ranks, op, nslices, **opts)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert guards_intact(slabs, dtype, x[0].size), "a kernel wrote outside the rank buffers"
    return [to_host(t, dtype) for t in slabs.ranks]


CASES = [(2, 37, 1), (3, 1000, 2), (5, 12345, 4), (8, 8 * 1024 + 5, 4), (16, 16 * 8 * 33 + 7, 5)]


@pytest.mark.parametrize("dtype,op", [("int32", "min"), ("int32", "prod"), ("fp32", "min"),
                                      ("fp32", "prod"), ("bf16", "min"), ("bf16", "prod"),
                                      ("fp16", "sum"), ("fp16", "max"), ("fp16", "min"),
                                      ("fp16", "prod")])
@pytest.mark.parametrize("R,count,nslices", CASES)
@pytest.mark.parametrize("sync", ["p2p", "barrier", "launch"])
def test_ops_small_ragged(rr, dtype, op, R, count, nslices, sync):
    log(f"case ops {dtype} {op} R={R} count={count} ns={nslices} sync={sync}")
    x = workloads.generate(R, count, dtype, _dist(dtype, op), R * 7 + count % 91)
    got = _run(rr, x, dtype, op, nslices, sync=sync)
    assert_matches_oracle(got, oracle_expect(x, op), dtype, f"{dtype} {op} R={R}")


@pytest.mark.parametrize("dtype,op", [("fp16", "sum"), ("fp16", "prod"), ("bf16", "prod"),
                                      ("int32", "prod"), ("fp32", "min")])
def test_ops_multi_tile(rr, dtype, op):
    R, count, ns = 8, (1 << 21) + 9, 8
    log(f"case ops multi {dtype} {op}")
    x = workloads.generate(R, count, dtype, _dist(dtype, op), 77)
    got = _run(rr, x, dtype, op, ns)
    assert_matches_oracle(got, oracle_expect(x, op), dtype, f"multi {dtype} {op}")


def test_fp16_specials_and_subnormals(rr):
    """Special values through the GPU fold: infinities, NaN (0x7E00 either side),
    overflow, subnormal sums and products, signed zeros."""
    pairs = [(0x7C00, 0x3C00), (0xFC00, 0x3C00), (0x7C00, 0xFC00), (0x7E01, 0x3C00),
             (0x7BFF, 0x7BFF), (0x7BFF, 0x4B80), (0x7BFF, 0x4C00), (0x0001, 0x0001),
             (0x8000, 0x8000), (0x3C00, 0xBC00), (0x0003, 0x3800), (0x03FF, 0x0001),
             (0x5C00, 0x5C00), (0x0200, 0x0200)]
    rng = np.random.default_rng(5)
    extra = rng.integers(0, 1 << 16, size=(4000, 2))
    extra = [(int(a), int(b)) for a, b in extra
             if ((a >> 10) & 0x1F) != 0x1F and ((b >> 10) & 0x1F) != 0x1F]
    allp = pairs + extra
    a = np.array([p[0] for p in allp], np.uint16).view(np.float16)
    b = np.array([p[1] for p in allp], np.uint16).view(np.float16)
    for op in ("sum", "prod", "max", "min"):
        log(f"case fp16 specials {op}")
        x = [a.copy(), b.copy()]
        got = _run(rr, x, "fp16", op, 1)
        assert_matches_oracle(got, oracle_expect(x, op), "fp16", f"fp16 specials {op}")


def test_ops_with_rounds_depth_and_fusion(rr):
    R, count, ns = 8, (1 << 20) + 13, 4
    x = workloads.generate(R, count, "fp16", "normal", 78)
    want = oracle_expect(x, "sum")
    for opts in (dict(sync="barrier", depth=2, rounds=2), dict(sync="p2p", fused=True),
                 dict(sync="barrier", depth=4, team=8, fused=True)):
        log(f"case fp16 {opts}")
        got = _run(rr, x, "fp16", "sum", ns, **opts)
        assert_matches_oracle(got, want, "fp16", f"fp16 {opts}")


def _special_pairs(dtype, rng):
    """Bit patterns that exercise the fold's edge cases, plus random bits (NaN and
    infinity patterns included) for the floating types."""
    if dtype == "fp32":
        inf, ninf, qnan, snan = 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001
        maxf, minsub, maxsub, one, mone = 0x7F7FFFFF, 0x00000001, 0x007FFFFF, 0x3F800000, 0xBF800000
        pairs = [(inf, one), (ninf, one), (inf, ninf), (qnan, one), (one, snan), (0xFFC12345, one),
                 (maxf, maxf), (maxf, 0x73800000), (minsub, minsub), (maxsub, minsub),
                 (0x80000000, 0x80000000), (0x80000000, 0), (one, mone), (0x00800000, 0x80000001),
                 (0x33800000, one), (0x33800001, one), (0x4B800000, 0x3F000000), (minsub, 0x3F000000)]
        extra = rng.integers(0, 1 << 32, size=(4000, 2), dtype=np.uint64)
        raw = np.uint32
    elif dtype == "bf16":
        inf, ninf, qnan = 0x7F80, 0xFF80, 0x7FC0
        pairs = [(inf, 0x3F80), (ninf, 0x3F80), (inf, ninf), (qnan, 0x3F80), (0x3F80, 0x7F81),
                 (0x7F7F, 0x7F7F), (0x7F7F, 0x7B00), (0x0001, 0x0001), (0x007F, 0x0001),
                 (0x8000, 0x8000), (0x8000, 0x0000), (0x3F80, 0xBF80), (0x3F80, 0x3B80),
                 (0x3F81, 0x3B80), (0x4380, 0x3F00), (0x0001, 0x3F00), (0x1000, 0x1000)]
        extra = rng.integers(0, 1 << 16, size=(4000, 2), dtype=np.uint64)
        raw = np.uint16
    else:
        imax, imin = 0x7FFFFFFF, 0x80000000
        pairs = [(imax, 1), (imin, 0xFFFFFFFF), (imax, imax), (imin, imin), (imax, imin),
                 (0x10000, 0x10000), (0xFFFFFFFF, 0xFFFFFFFF), (0, imin), (46341, 46341)]
        extra = rng.integers(0, 1 << 32, size=(4000, 2), dtype=np.uint64)
        raw = np.uint32
    allp = pairs + [(int(a), int(b)) for a, b in extra]
    a = np.array([p[0] for p in allp], dtype=np.uint64).astype(raw)
    b = np.array([p[1] for p in allp], dtype=np.uint64).astype(raw)
    view = {"fp32": np.float32, "bf16": np.uint16, "int32": np.int32}[dtype]
    return a.view(view), b.view(view), raw


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "int32"])
@pytest.mark.parametrize("R", [2, 3])
def test_specials_through_the_ring(rr, dtype, R):
    """Special values through the ring's folds, bit for bit against the oracle:
    infinities, NaN (fp32 compared as "both NaN", bf16 canonical 0x7FC0),
    overflow to infinity, subnormal operands and results (kept, not flushed),
    signed zeros, rounding ties, and int32 wrap-around in SUM and PROD.  With
    R = 3 the chunk values pass through two folds."""
    rng = np.random.default_rng(11 + R)
    a, b, raw = _special_pairs(dtype, rng)
    x = [a.copy(), b.copy()]
    if R == 3:
        x.append(rng.permutation(b).copy())
    for op in ("sum", "prod", "max", "min"):
        log(f"case specials {dtype} R={R} {op}")
        got = _run(rr, [t.copy() for t in x], dtype, op, 1)
        assert_matches_oracle(got, oracle_expect([t.copy() for t in x], op), dtype,
                              f"specials {dtype} R={R} {op}")


@pytest.mark.parametrize("op", ["sum", "prod", "max", "min"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_16bit_operand_pairs_through_the_hop(rr, dtype, op):
    """Every 32nd 16-bit pattern as first operand against all 65536 as second
    (134 million ordered pairs: every sign, zero, subnormal, infinity and NaN
    class on both sides) through one fold of the ring on the GPU, bit for bit
    against the oracle, whose folds are pinned on all 2^32 pairs on the CPU.
    R = 2: rank 0 holds the first operands and rank 1 the second ones; each
    position is folded once (rank 0's value into rank 1's in the first chunk,
    the other way in the second) and both ranks end with the result."""
    firsts = np.arange(0, 1 << 16, 32, dtype=np.uint16)
    a = np.repeat(firsts, 1 << 16)
    b = np.tile(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16), firsts.size)
    x = [a, b] if dtype == "bf16" else [a.view(np.float16), b.view(np.float16)]
    log(f"case 16-bit pairs {dtype} {op}: {a.size} pairs")
    slabs = to_slabs(rr, x, dtype)
    rr.allreduce_ring(slabs.ranks, op, 1)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert guards_intact(slabs, dtype, a.size), "a kernel wrote outside the rank buffers"
    want = oracle_expect(x, op)
    assert_full_matches(slabs.ranks, want, dtype, f"16-bit pairs {dtype} {op}")


@pytest.mark.parametrize("op", ["sum", "prod", "max", "min"])
@pytest.mark.parametrize("dtype", ["fp32", "int32"])
def test_32bit_random_patterns_through_the_hop(rr, dtype, op):
    """64 million ordered pairs of uniformly random 32-bit patterns (for fp32:
    every class -- normal, subnormal, zero, infinity, NaN with any payload --
    in proportion to its share of the patterns) through one fold of the ring on
    the GPU, against the oracle (fp32 NaNs compare as NaN whatever the payload).
    R = 2, as in the 16-bit test above."""
    rng = np.random.default_rng(4242 + len(op))
    a = rng.integers(0, 1 << 32, size=1 << 26, dtype=np.uint64).astype(np.uint32)
    b = rng.integers(0, 1 << 32, size=1 << 26, dtype=np.uint64).astype(np.uint32)
    view = np.float32 if dtype == "fp32" else np.int32
    x = [a.view(view), b.view(view)]
    log(f"case 32-bit patterns {dtype} {op}: {a.size} pairs")
    slabs = to_slabs(rr, x, dtype)
    rr.allreduce_ring(slabs.ranks, op, 1)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    assert guards_intact(slabs, dtype, a.size), "a kernel wrote outside the rank buffers"
    assert_full_matches(slabs.ranks, oracle_expect(x, op), dtype, f"32-bit patterns {dtype} {op}")
