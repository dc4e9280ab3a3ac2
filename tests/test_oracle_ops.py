"""Pins of the oracle's fp16 arithmetic and its MIN and PROD reductions (no GPU).

Against things other than the oracle itself:
* exact rational arithmetic and a round-to-nearest-even written from the IEEE
  754 definition (oracle/brute.py) on tiny inputs and on many single additions
  and multiplications;
* closed forms of tracer inputs (the MIN of ranks, products of known factors);
* special values fixed by IEEE 754 (infinities, NaN, overflow, subnormals).
The fold order is the ring's (the loosp.cn post, section 5): chunk c folds ranks
c, c+1, ... in turn, so these reductions take the same path as SUM and MAX.
"""
import random

import numpy as np
import pytest

import oracle
from oracle import brute
import workloads

RAW = {"int32": None, "fp32": np.uint32, "bf16": np.uint16, "fp16": np.uint16}
DIST = {("int32", "sum"): "int_pm1000", ("int32", "max"): "int_pm1000",
        ("int32", "min"): "int_pm1000", ("int32", "prod"): "unit_jitter"}


def _dist(dtype, op):
    if dtype == "int32":
        return DIST[(dtype, op)]
    return "unit_jitter" if op == "prod" else ("normal" if dtype != "fp32" else "uniform_pm1")


def _bits(a, dtype):
    if dtype == "int32":
        return a.astype(np.int64)
    return a.view(RAW[dtype]).astype(np.int64)


def _brute_expect(x, dtype, op, start_of=None):
    """Per position: the brute-force fold, starting at the chunk's own rank
    (or at start_of(position) when given)."""
    R, count = len(x), x[0].size
    bounds = oracle.chunk_bounds(count, R, dtype)
    out = np.empty(count, dtype=np.int64)
    for i in range(count):
        c = int(np.searchsorted(bounds, i, side="right") - 1) if start_of is None else start_of(i)
        vals = [int(x[r][i]) if dtype == "int32" else int(x[r].view(RAW[dtype])[i])
                for r in range(R)]
        out[i] = brute.allreduce_element(vals, c, dtype, op)
    return out


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16", "fp16"])
@pytest.mark.parametrize("op", ["min", "prod"])
@pytest.mark.parametrize("R,count", [(2, 9), (3, 40), (5, 37), (8, 70), (16, 100)])
def test_min_prod_brute_force(dtype, op, R, count):
    x = workloads.generate(R, count, dtype, _dist(dtype, op), 31 + R)
    bufs = [a.copy() for a in x]
    oracle.allreduce(bufs, op)
    expect = _brute_expect(x, dtype, op)
    for b in bufs:
        assert np.array_equal(_bits(b, dtype), expect)


@pytest.mark.parametrize("op", ["sum", "max"])
@pytest.mark.parametrize("R,count", [(2, 9), (4, 64), (7, 50), (16, 100)])
def test_fp16_sum_max_brute_force(op, R, count):
    x = workloads.generate(R, count, "fp16", "normal", 51 + R)
    bufs = [a.copy() for a in x]
    oracle.allreduce(bufs, op)
    expect = _brute_expect(x, "fp16", op)
    for b in bufs:
        assert np.array_equal(_bits(b, "fp16"), expect)


def test_min_of_rank_and_products_closed_form():
    R, count = 8, 8 * 4 * 3 + 1
    # MIN of "rank r holds r" is 0, MAX is R - 1, for every dtype
    for dtype in ("int32", "fp32", "bf16", "fp16"):
        x = workloads.generate(R, count, dtype, "rank", 0)
        a = [v.copy() for v in x]
        oracle.allreduce(a, "min")
        for b in a:
            assert np.all(b.astype(np.float64) == 0) if dtype != "bf16" else np.all(b == 0)
    # int32 product of 2..R+1 is (R+1)!; of 3 at 21 ranks wraps modulo 2^32
    x = [np.full(count, r + 2, np.int32) for r in range(R)]
    oracle.allreduce(x, "prod")
    assert np.all(x[3] == 362880)
    y = [np.full(17, 3, np.int32) for _ in range(21)]
    oracle.allreduce(y, "prod")
    want = (3 ** 21) % (1 << 32)
    want = want - (1 << 32) if want >= (1 << 31) else want
    assert np.all(y[0] == want)
    # fp32 product of powers of two is exact: 2^(sum of exponents)
    e = [np.full(count, 2.0 ** (r - 3), np.float32) for r in range(R)]
    oracle.allreduce(e, "prod")
    assert np.all(e[5] == np.float32(2.0 ** sum(r - 3 for r in range(R))))


def _fp16_pairs(n, seed):
    rnd = random.Random(seed)
    special = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x3C00,
               0xBC00, 0x3C01, 0x4000, 0x7800, 0x0200, 0x5BFF, 0x1400]
    pairs = [(a, b) for a in special for b in special]
    while len(pairs) < n:
        a = rnd.getrandbits(16)
        if rnd.random() < 0.5:
            e = (a >> 10) & 0x1F
            e2 = max(0, min(30, e + rnd.randint(-6, 6)))
            b = (rnd.getrandbits(1) << 15) | (e2 << 10) | rnd.getrandbits(10)
        else:
            b = rnd.getrandbits(16)
        if ((a >> 10) & 0x1F) == 0x1F or ((b >> 10) & 0x1F) == 0x1F:
            continue
        pairs.append((a, b))
    return pairs


@pytest.mark.parametrize("op", ["sum", "prod"])
def test_fp16_hop_is_correctly_rounded(op, n=20000):
    """Each fp16 hop equals the exact result rounded once to binary16."""
    pairs = _fp16_pairs(n, 7 if op == "sum" else 8)
    a = np.array([p[0] for p in pairs], dtype=np.uint16).view(np.float16)
    b = np.array([p[1] for p in pairs], dtype=np.uint16).view(np.float16)
    bufs = [a.copy(), b.copy()]
    oracle.allreduce(bufs, op)  # R = 2: one operation per element
    f = brute.add if op == "sum" else brute.mul
    for k, (pa, pb) in enumerate(pairs):
        want = brute.value_to_fp16_bits(
            f(brute.fp16_bits_to_value(pa), brute.fp16_bits_to_value(pb), "fp16"))
        got = int(bufs[0].view(np.uint16)[k])
        assert got == want and int(bufs[1].view(np.uint16)[k]) == want, (hex(pa), hex(pb))


def test_fp16_special_values():
    inf, ninf, nan = 0x7C00, 0xFC00, 0x7E01
    sums = [(inf, 0x3C00, inf), (ninf, 0x3C00, ninf), (inf, ninf, 0x7E00), (nan, 0x3C00, 0x7E00),
            (0x7BFF, 0x7BFF, inf),           # 65504 + 65504 overflows
            (0x7BFF, 0x4B80, 0x7BFF),        # 65504 + 15 = 65519 rounds down
            (0x7BFF, 0x4C00, inf),           # 65504 + 16 = 65520 is the tie: to even -> inf
            (0x0001, 0x0001, 0x0002),        # subnormals add exactly
            (0x8000, 0x8000, 0x8000), (0x3C00, 0xBC00, 0x0000)]
    a = np.array([c[0] for c in sums], np.uint16).view(np.float16)
    b = np.array([c[1] for c in sums], np.uint16).view(np.float16)
    bufs = [a.copy(), b.copy()]
    oracle.allreduce(bufs, "sum")
    assert [int(v) for v in bufs[0].view(np.uint16)] == [c[2] for c in sums]
    prods = [(inf, 0x0000, 0x7E00), (0x0001, 0x3800, 0x0000),   # 2^-24 * 0.5: tie to even 0
             (0x0003, 0x3800, 0x0002),                          # 1.5 * 2^-24: tie to even 2
             (0x5BFF, 0x5BFF, 0x7BFE),                          # 255.875^2 = 65472.02 -> 65472
             (0x5C00, 0x5C00, inf),                             # 256^2 = 65536 overflows
             (0xBC00, 0x0000, 0x8000)]
    a = np.array([c[0] for c in prods], np.uint16).view(np.float16)
    b = np.array([c[1] for c in prods], np.uint16).view(np.float16)
    bufs = [a.copy(), b.copy()]
    oracle.allreduce(bufs, "prod")
    assert [int(v) for v in bufs[0].view(np.uint16)] == [c[2] for c in prods]


def test_bf16_product_is_correctly_rounded(n=20000):
    """bf16 PROD is the exact product rounded once to bf16.  The GPU computes
    the binary32 product and rounds that to bf16; the brute force checks on
    the same pairs (subnormal and overflowing products included) that the two
    roundings give the same bits, as they must: a product of two bf16 values
    has at most 16 significant bits, too few for the binary32 rounding to
    create a tie at 8 bits."""
    rnd = random.Random(3)
    pairs = [(rnd.getrandbits(16), rnd.getrandbits(16)) for _ in range(n)]
    pairs = [(p, q) for p, q in pairs if ((p >> 7) & 0xFF) != 0xFF and ((q >> 7) & 0xFF) != 0xFF]
    a = np.array([p[0] for p in pairs], np.uint16)
    b = np.array([p[1] for p in pairs], np.uint16)
    bufs = [a.copy(), b.copy()]
    oracle.allreduce(bufs, "prod")
    for k, (pa, pb) in enumerate(pairs):
        va, vb = brute.bf16_bits_to_value(pa), brute.bf16_bits_to_value(pb)
        want = brute.value_to_bf16_bits(brute.mul(va, vb, "bf16"))
        two_step = brute.mul(va, vb, "fp32")
        if not isinstance(two_step, float):
            r = brute.round_nearest_even(two_step, "bf16")
            two_step = (-0.0 if two_step < 0 else 0.0) if r == 0 else r
        assert brute.value_to_bf16_bits(two_step) == want, (hex(pa), hex(pb))
        assert int(bufs[0][k]) == want, (hex(pa), hex(pb))


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16", "fp16"])
def test_min_max_take_an_input(dtype):
    """MIN and MAX do no arithmetic: every result is one of the ranks' inputs."""
    R, count = 6, 6 * 8 + 5
    x = workloads.generate(R, count, dtype, "normal" if dtype != "int32" else "int_pm1000", 9)
    for op in ("min", "max"):
        a = [v.copy() for v in x]
        oracle.allreduce(a, op)
        raw = [_bits(v, dtype) for v in x]
        got = _bits(a[0], dtype)
        for i in range(count):
            assert any(int(got[i]) == int(raw[r][i]) for r in range(R))
