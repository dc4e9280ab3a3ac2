"""Pins of the CPU oracle to things other than itself (no GPU needed).

* the worked 4-GPU example and the primitive table of the post "Why AllReduce =
  ReduceScatter + AllGather -- with NCCL Ring AllReduce" (fixtures under
  tests/golden/);
* closed forms of provenance-tagged integer inputs;
* brute force with exact rational arithmetic on tiny inputs (oracle/brute.py);
* invariants: AllGather is a bit copy, ReduceScatter then AllGather equals
  AllReduce, per-rank traffic equals the post's 2N(k-1)/k (section 13);
* the floating-point error bounds that the ring's fold order must meet.
"""
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
import workloads

LETTERS = "abcdefghijklmnopqrstuvwxyz"


def _parse_worked_example(path):
    rs, own, ag, final = [], {}, [], {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            p = line.split()
            if p[0] == "RS":
                terms = tuple(LETTERS.index(t[0]) for t in p[5].split("+"))
                chunks = {int(t[1:]) for t in p[5].split("+")}
                assert chunks == {int(p[4])}
                rs.append((int(p[1]), int(p[2]), int(p[3]), int(p[4]), terms))
            elif p[0] == "OWN":
                own[int(p[1])] = int(p[2])
            elif p[0] == "AG":
                ag.append((int(p[1]), int(p[2]), int(p[3]), None if p[4] == "?" else int(p[4])))
            elif p[0] == "FINAL":
                final[int(p[1])] = [int(c) for c in p[2].split(",")]
    return rs, own, ag, final


def test_worked_example_schedule(golden_dir):
    rs, own, ag, final = _parse_worked_example(os.path.join(golden_dir, "worked_example_r4.txt"))
    w = workloads.WORKED_EXAMPLE
    bufs = workloads.inputs(w)
    hops = oracle.allreduce(bufs, "sum", trace=True)
    got_rs = {(h.round, h.src): h for h in hops if h.phase == "RS"}
    assert len(got_rs) == len(rs) == 12
    for rnd, src, dst, chunk, terms in rs:
        h = got_rs[(rnd, src)]
        assert (h.dst, h.chunk, h.terms) == (dst, chunk, terms), (rnd, src)
    # ownership: the finished chunk sits where the last ReduceScatter round left it
    last = {h.dst: h for h in hops if h.phase == "RS" and h.round == 3}
    for rank, chunk in own.items():
        assert last[rank].chunk == chunk and len(last[rank].terms) == 4
    got_ag = {(h.round, h.src): h for h in hops if h.phase == "AG"}
    assert len(got_ag) == len(ag) == 12
    for rnd, src, dst, chunk in ag:
        h = got_ag[(rnd, src)]
        assert h.dst == dst
        if chunk is not None:
            assert h.chunk == chunk
        assert len(h.terms) == 4  # AllGather only moves finished chunks
    # Round 3 (chunk labels absent on the page): each rank forwards what it got in round 2
    for src in range(4):
        assert got_ag[(3, src)].chunk == got_ag[(2, (src - 1) % 4)].chunk
    # final state: every rank received every chunk other than the one it finished
    held = {r: {own[r]} for r in range(4)}
    for h in hops:
        if h.phase == "AG":
            held[h.dst].add(h.chunk)
    for rank, chunks in final.items():
        assert sorted(held[rank]) == chunks


def test_worked_example_values():
    """Section 1: every GPU ends with [S0..S3], S_k the sum of the ranks' chunk k."""
    w = workloads.WORKED_EXAMPLE
    x = workloads.inputs(w)
    bufs = [a.copy() for a in x]
    oracle.allreduce(bufs, "sum")
    expect = np.sum(np.stack([a.astype(np.int64) for a in x]), axis=0)
    for b in bufs:
        assert np.array_equal(b.astype(np.int64), expect)


def test_table_v_k4(golden_dir):
    want = []
    with open(os.path.join(golden_dir, "table_v_k4.txt"), encoding="utf-8") as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                want.append(line.split()[1])
    bufs = workloads.generate(4, 64, "int32", "int_pm1000", 1)
    labels = oracle.primitive_labels(oracle.allreduce(bufs, trace=True), 4)
    for rank in range(4):
        assert labels[rank] == want


@pytest.mark.parametrize("R", [2, 3, 5, 8, 16])
def test_table_v_general(R):
    bufs = workloads.generate(R, 8 * R, "fp32", "uniform_pm1", 7)
    hops = oracle.allreduce(bufs, trace=True)
    assert len({h.hop for h in hops}) == 2 * (R - 1)          # ring rounds
    want = (["send"] + ["recvReduceSend"] * (R - 2) + ["recvReduceCopySend"]
            + ["recvCopySend"] * (R - 2) + ["recv"])
    labels = oracle.primitive_labels(hops, R)
    for rank in range(R):
        assert labels[rank] == want and len(want) == 2 * R - 1


@pytest.mark.parametrize("R,count", [(4, 64), (8, 1024), (16, 16 * 40), (7, 7 * 12)])
def test_volume_per_rank(R, count):
    """Section 13: each rank sends N(k-1)/k in each phase, 2N(k-1)/k in all."""
    bufs = workloads.generate(R, count, "fp32", "uniform_pm1", 3)
    hops = oracle.allreduce(bufs, trace=True)
    N = count * 4
    for rank in range(R):
        rs = sum(h.bytes for h in hops if h.src == rank and h.phase == "RS")
        ag = sum(h.bytes for h in hops if h.src == rank and h.phase == "AG")
        assert rs == ag == N * (R - 1) // R


@pytest.mark.parametrize("R", [2, 4, 8, 16, 31])
def test_onehot_tracer(R):
    """Rank r contributes 1 << r: a missing or doubled hop flips a bit."""
    count = 4 * R + 3
    bufs = workloads.generate(R, count, "int32", "onehot", 0)
    oracle.allreduce(bufs, "sum")
    for b in bufs:
        assert np.all(b == (1 << R) - 1 if R < 31 else b == np.int32((1 << 31) - 1))


@pytest.mark.parametrize("R", [2, 3, 8, 16, 64])
def test_rank_index_closed_form(R):
    count = 4 * R * 3 + 1
    bufs = workloads.generate(R, count, "int32", "rank_index", 0)
    oracle.allreduce(bufs, "sum")
    i = np.arange(count, dtype=np.int64)
    expect = 1000 * R * (R - 1) // 2 + R * i
    for b in bufs:
        assert np.array_equal(b.astype(np.int64), expect)


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
def test_max_of_rank(dtype):
    R = 9
    bufs = workloads.generate(R, 100, "int32", "rank", 0)
    if dtype != "int32":
        bufs = [workloads._as_dtype(b.astype(np.float32), dtype) for b in bufs]
    oracle.allreduce(bufs, "max")
    top = workloads._as_dtype(np.array([R - 1], dtype=np.float32 if dtype != "int32" else np.int32),
                              dtype)[0]
    for b in bufs:
        assert np.all(b == top)


def _brute_expect(x, dtype, op):
    R, count = len(x), x[0].size
    bounds = oracle.chunk_bounds(count, R, dtype)
    out = np.empty(count, dtype=np.int64)
    for i in range(count):
        c = int(np.searchsorted(bounds, i, side="right") - 1)
        vals = [int(x[r][i]) if dtype == "int32" else int(x[r].view(
            np.uint32 if dtype == "fp32" else np.uint16)[i]) for r in range(R)]
        out[i] = brute.allreduce_element(vals, c, dtype, op)
    return out


def _bits(a, dtype):
    if dtype == "int32":
        return a.astype(np.int64)
    return a.view(np.uint32 if dtype == "fp32" else np.uint16).astype(np.int64)


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
@pytest.mark.parametrize("op", ["sum", "max"])
@pytest.mark.parametrize("R,count", [(2, 9), (3, 40), (4, 64), (5, 37), (8, 70), (6, 3), (16, 100)])
def test_brute_force_tiny(dtype, op, R, count):
    dist = {"int32": "int_pm1000", "fp32": "uniform_pm1", "bf16": "normal"}[dtype]
    x = workloads.generate(R, count, dtype, dist, 11 + R)
    bufs = [a.copy() for a in x]
    oracle.allreduce(bufs, op)
    expect = _brute_expect(x, dtype, op)
    for b in bufs:
        assert np.array_equal(_bits(b, dtype), expect)


def test_fold_order_is_the_rings():
    """fp32 values chosen so that the result depends on the fold order.

    In chunk c the ring adds ranks c, c+1, ... in turn.  Rank 0 holds 1.0 and
    ranks 1..3 hold t = 2^-24 (half an ulp of 1.0).  Adding t to 1.0 is a tie
    that rounds back to 1.0 (even), 2t = 2^-23 is exactly one ulp, and 1 + 3t is
    a tie that rounds up to 1 + 4t (even).  So:
      chunk 0: ((1 + t) + t) + t      -> 1.0
      chunk 1: ((t + t) + t) + 1      -> 1 + 3t -> 1 + 2^-22
      chunk 2: ((t + t) + 1) + t      -> (1 + 2t) + t -> 1 + 2^-22
      chunk 3: ((t + 1) + t) + t      -> 1.0
    Any other fold order gives a different pattern.
    """
    R = 4
    count = 16  # 4 chunks of one 16-byte vector
    x = [np.zeros(count, np.float32) for _ in range(R)]
    tiny = np.float32(2.0 ** -24)
    for r in range(1, R):
        x[r][:] = tiny
    x[0][:] = 1.0
    bufs = [a.copy() for a in x]
    oracle.allreduce(bufs, "sum")
    bounds = oracle.chunk_bounds(count, R, "fp32")
    for c in range(R):
        lo, hi = int(bounds[c]), int(bounds[c + 1])
        want = np.float32(1.0) if c in (0, 3) else np.float32(1.0 + 2.0 ** -22)
        for b in bufs:
            assert np.all(b[lo:hi] == want), c
    # and the brute-force reference agrees on the same positions
    assert np.array_equal(_bits(bufs[0], "fp32"), _brute_expect(x, "fp32", "sum"))


def _bf16_pairs(n, seed):
    rnd = random.Random(seed)
    pairs = []
    special = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x3F80,
               0xBF80, 0x3F81, 0x4000, 0x7F00, 0x0100]
    for a in special:
        for b in special:
            pairs.append((a, b))
    while len(pairs) < n:
        a = rnd.getrandbits(16)
        # partner with a nearby exponent half of the time, so sums need rounding
        if rnd.random() < 0.5:
            e = (a >> 7) & 0xFF
            e2 = max(0, min(254, e + rnd.randint(-10, 10)))
            b = (rnd.getrandbits(1) << 15) | (e2 << 7) | rnd.getrandbits(7)
        else:
            b = rnd.getrandbits(16)
        ea, eb = (a >> 7) & 0xFF, (b >> 7) & 0xFF
        if ea == 0xFF or eb == 0xFF:
            continue  # inf and NaN are checked separately below
        pairs.append((a, b))
    return pairs


def test_bf16_add_is_correctly_rounded():
    """Every bf16 hop equals the exact sum rounded once to bf16 (ties to even)."""
    pairs = _bf16_pairs(40000, 5)
    a = np.array([p[0] for p in pairs], dtype=np.uint16)
    b = np.array([p[1] for p in pairs], dtype=np.uint16)
    bufs = [a.copy(), b.copy()]
    oracle.allreduce(bufs, "sum")  # R=2: every element is one addition
    for k, (pa, pb) in enumerate(pairs):
        want = brute.value_to_bf16_bits(
            brute.add(brute.bf16_bits_to_value(pa), brute.bf16_bits_to_value(pb), "bf16"))
        assert int(bufs[0][k]) == want and int(bufs[1][k]) == want, (hex(pa), hex(pb))


def test_bf16_special_values():
    inf, ninf, nan = 0x7F80, 0xFF80, 0x7FC1
    cases = [(inf, 0x3F80, inf), (ninf, 0x3F80, ninf), (inf, ninf, 0x7FC0), (nan, 0x3F80, 0x7FC0),
             (0x7F7F, 0x7F7F, inf), (0x8000, 0x8000, 0x8000), (0x3F80, 0xBF80, 0x0000)]
    a = np.array([c[0] for c in cases], np.uint16)
    b = np.array([c[1] for c in cases], np.uint16)
    bufs = [a, b]
    oracle.allreduce(bufs, "sum")
    assert [int(v) for v in bufs[0]] == [c[2] for c in cases]


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
@pytest.mark.parametrize("R", [2, 5, 8])
def test_all_gather_is_a_bit_copy(dtype, R):
    """Section 6: AllGather does no arithmetic, so NaN payloads survive."""
    count = 4 * R * 5 + 3
    x = workloads.generate(R, count, dtype, "bits", 21)
    bufs = [a.copy() for a in x]
    oracle.all_gather(bufs)
    bounds = oracle.chunk_bounds(count, R, dtype)
    raw = np.uint32 if dtype != "bf16" else np.uint16
    for c in range(R):
        lo, hi = int(bounds[c]), int(bounds[c + 1])
        owner = (c - 1) % R
        src = x[owner].view(raw)[lo:hi]
        for b in bufs:
            assert np.array_equal(b.view(raw)[lo:hi], src)


@pytest.mark.parametrize("dtype,op", [("int32", "sum"), ("fp32", "sum"), ("bf16", "sum"),
                                      ("fp32", "max"), ("bf16", "max")])
@pytest.mark.parametrize("R", [2, 3, 8])
def test_reduce_scatter_then_all_gather(dtype, op, R):
    count = 8 * R * 3 + 5
    dist = {"int32": "int_pm1000", "fp32": "uniform_pm1", "bf16": "normal"}[dtype]
    x = workloads.generate(R, count, dtype, dist, 4)
    a = [v.copy() for v in x]
    b = [v.copy() for v in x]
    oracle.allreduce(a, op)
    oracle.reduce_scatter(b, op)
    bounds = oracle.chunk_bounds(count, R, dtype)
    raw = np.uint32 if dtype != "bf16" else np.uint16
    for r in range(R):  # rank r owns chunk (r + 1) mod R after ReduceScatter
        c = (r + 1) % R
        lo, hi = int(bounds[c]), int(bounds[c + 1])
        assert np.array_equal(b[r].view(raw)[lo:hi], a[r].view(raw)[lo:hi])
    oracle.all_gather(b)
    for r in range(R):
        assert np.array_equal(a[r].view(raw), b[r].view(raw))


def test_reduce_scatter_partials():
    """After ReduceScatter chunk c of rank r folds ranks c .. r (section 5)."""
    R, count = 5, 5 * 4
    x = workloads.generate(R, count, "int32", "onehot", 0)
    bufs = [v.copy() for v in x]
    oracle.reduce_scatter(bufs, "sum")
    bounds = oracle.chunk_bounds(count, R, "int32")
    for r in range(R):
        for c in range(R):
            n = (r - c) % R + 1
            mask = sum(1 << ((c + k) % R) for k in range(n))
            lo, hi = int(bounds[c]), int(bounds[c + 1])
            assert np.all(bufs[r][lo:hi] == mask), (r, c)


@pytest.mark.parametrize("count,R,dtype", [(0, 4, "fp32"), (1, 4, "fp32"), (10, 4, "fp32"),
                                           (64, 4, "int32"), (100, 8, "bf16"), (3, 64, "fp32"),
                                           (1 << 20, 16, "fp32"), (17, 1, "int32")])
def test_partition(count, R, dtype):
    b = oracle.chunk_bounds(count, R, dtype)
    v = 16 // workloads.ELEM_BYTES[dtype]
    assert b[0] == 0 and b[-1] == count
    assert np.all(np.diff(b.astype(np.int64)) >= 0)
    nominal = -(-(-(-count // R)) // v) * v  # ceil(count / R) rounded up to a vector
    for c in range(R):
        assert b[c] == min(c * nominal, count)
        assert b[c] % v == 0 or b[c] == count
    # the chunks cover [0, count) with at most one partial chunk
    sizes = np.diff(b.astype(np.int64))
    assert sizes.sum() == count
    assert np.count_nonzero((sizes > 0) & (sizes < nominal)) <= 1


def test_edge_cases():
    x = workloads.generate(1, 33, "fp32", "uniform_pm1", 1)
    y = [x[0].copy()]
    oracle.allreduce(y)
    assert np.array_equal(x[0], y[0])  # one rank: nothing to do
    z = [np.zeros(0, np.float32) for _ in range(4)]
    oracle.allreduce(z)  # empty: no-op
    # fewer elements than ranks: trailing chunks are empty, result still exact
    x = workloads.generate(8, 5, "int32", "int_pm1000", 2)
    bufs = [v.copy() for v in x]
    oracle.allreduce(bufs)
    s = np.sum(np.stack(x).astype(np.int64), axis=0)
    for b in bufs:
        assert np.array_equal(b.astype(np.int64), s)


def test_int32_wraps():
    R = 4
    x = [np.full(8, 2 ** 31 - 1, dtype=np.int32) for _ in range(R)]
    oracle.allreduce(x)
    want = ((2 ** 31 - 1) * R) & 0xFFFFFFFF
    want = want - 2 ** 32 if want >= 2 ** 31 else want
    assert np.all(x[0] == want)


def test_fp32_error_bound_r64():
    """Ring fp32 sum stays within (R-1)u/(1-(R-1)u) * sum|x| of the exact sum."""
    R, count = 64, 4 * 64 * 8
    x = workloads.generate(R, count, "fp32", "uniform_pm1", 9)
    d, a = oracle.direct_sum_f64(x)
    bufs = [v.copy() for v in x]
    oracle.allreduce(bufs)
    u = 2.0 ** -24
    gamma = (R - 1) * u / (1 - (R - 1) * u)
    err = np.abs(bufs[0].astype(np.float64) - d)
    assert np.all(err <= gamma * a + 1e-300)
    assert np.all(err <= 1e-5 * a)
    assert np.any(err > 0)  # the fold really rounds


def test_bf16_error_bound_r8():
    R, count = 8, 8 * 8 * 64
    x = workloads.generate(R, count, "bf16", "normal", 3)
    d, a = oracle.direct_sum_f64(x)
    bufs = [v.copy() for v in x]
    oracle.allreduce(bufs)
    y = (bufs[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rel = np.linalg.norm(y - d) / np.linalg.norm(d)
    assert rel <= 1e-2
    u = 2.0 ** -8
    gamma = (R - 1) * u / (1 - (R - 1) * u)
    assert np.all(np.abs(y - d) <= gamma * a * (1 + 1e-12))


@pytest.mark.parametrize("dtype,op", [("fp32", "sum"), ("bf16", "sum"), ("int32", "sum"),
                                      ("fp32", "max")])
def test_allreduce_at_matches_full_run(dtype, op):
    R, count = 8, 8 * 8 * 10 + 3
    dist = {"int32": "int_pm1000", "fp32": "uniform_pm1", "bf16": "normal"}[dtype]
    x = workloads.generate(R, count, dtype, dist, 6)
    full = [v.copy() for v in x]
    oracle.allreduce(full, op)
    bounds = oracle.chunk_bounds(count, R, dtype)
    pos = np.array([0, 1, count - 1, count // 2, int(bounds[3]), int(bounds[3]) - 1, 77])
    chunks = np.searchsorted(bounds, pos, side="right") - 1
    vals = np.stack([x[r][pos] for r in range(R)], axis=1)
    got = oracle.allreduce_at(vals, chunks, dtype, op)
    for k, p in enumerate(pos):
        for r in range(R):
            assert _bits(got[k:k + 1, r], dtype)[0] == _bits(full[r][p:p + 1], dtype)[0]


# ------------------------------------------- the order-free reference sum
# ro_direct_sum_f64 gives, per element, the sum of the ranks' values and of
# their magnitudes, accumulated in binary64 in rank order.  It is the expected
# value of every floating-point tolerance check (the ring post, section 1: the
# AllReduce result is the reduction over all ranks), so it is pinned here to
# the formats' own decoding, to exact rational sums and to math.fsum.

def _decode_exact(bits, dtype):
    """Exact value of one pattern: a Fraction, or a float for zero, inf, NaN."""
    if dtype == "bf16":
        return brute.bf16_bits_to_value(int(bits))
    if dtype == "fp16":
        return brute.fp16_bits_to_value(int(bits))
    return brute.fp32_bits_to_value(int(bits))


def _as_float(v):
    return v if isinstance(v, float) else float(v)


def _raw(dtype, bits):
    bits = np.asarray(bits)
    if dtype == "bf16":
        return bits.astype(np.uint16)
    if dtype == "fp16":
        return bits.astype(np.uint16).view(np.float16)
    return bits.astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_direct_sum_decodes_every_16bit_pattern(dtype):
    """One rank: the sum is the pattern's value and the magnitude sum its
    absolute value, for all 65536 patterns (subnormals, infinities and NaNs
    included), each decoded exactly by the brute-force module."""
    x = _raw(dtype, np.arange(1 << 16))
    s, a = oracle.direct_sum_f64([x])
    for bits in range(1 << 16):
        v = _decode_exact(bits, dtype)
        if isinstance(v, float) and v != v:
            assert np.isnan(s[bits]) and np.isnan(a[bits]), hex(bits)
            continue
        want = _as_float(v)
        assert s[bits] == want and a[bits] == abs(want), (hex(bits), s[bits], want)


def test_direct_sum_decodes_fp32_patterns():
    """One rank, binary32: subnormals, the extremes, specials and random bits."""
    rnd = random.Random(12)
    pats = [0x00000001, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x80000001, 0xFF7FFFFF, 0x3F800000,
            0x7F800000, 0xFF800000, 0x7FC00001, 0x80000000] + [rnd.getrandbits(32) for _ in range(4000)]
    x = _raw("fp32", pats)
    s, a = oracle.direct_sum_f64([x])
    for k, bits in enumerate(pats):
        v = _decode_exact(bits, "fp32")
        if isinstance(v, float) and v != v:
            assert np.isnan(s[k])
            continue
        assert s[k] == _as_float(v) and a[k] == abs(_as_float(v)), hex(bits)


@pytest.mark.parametrize("dtype,dist,R", [("fp32", "uniform_pm1", 64), ("bf16", "normal", 8),
                                          ("fp16", "normal", 8), ("fp32", "uniform_pm1", 3)])
def test_direct_sum_is_the_exact_sum(dtype, dist, R):
    """On the workloads' value distributions every partial sum fits binary64's
    53 bits, so the result must be the exact rational sum (checked to be
    representable first), and equal to math.fsum; the magnitude sum likewise."""
    count = 700
    x = workloads.generate(R, count, dtype, dist, 77 + R)
    s, a = oracle.direct_sum_f64(x)
    raw = [v.view(np.uint16) if dtype != "fp32" else v.view(np.uint32) for v in x]
    for i in range(count):
        vals = [_decode_exact(raw[r][i], dtype) for r in range(R)]
        fr = [v if not isinstance(v, float) else Fraction(0) for v in vals]
        exact = sum(fr, Fraction(0))
        mag = sum((abs(v) for v in fr), Fraction(0))
        assert Fraction(float(exact)) == exact and Fraction(float(mag)) == mag
        assert s[i] == float(exact), (i, s[i], float(exact))
        assert a[i] == float(mag)
        assert s[i] == math.fsum(float(v) for v in fr)


@pytest.mark.parametrize("dtype,small", [("fp32", 0x30800000), ("bf16", 0x3080), ("fp16", 0x0001)])
def test_direct_sum_keeps_far_apart_terms(dtype, small):
    """1 + tiny - 1 with tiny far below the format's unit at 1 (2^-30, or
    binary16's smallest subnormal 2^-24): exact in binary64, lost by any
    narrower accumulator; 1 - 1 + tiny gives the same; magnitudes add."""
    one, mone = {"fp32": (0x3F800000, 0xBF800000), "bf16": (0x3F80, 0xBF80),
                 "fp16": (0x3C00, 0xBC00)}[dtype]
    tiny = _as_float(_decode_exact(small, dtype))
    for order in ((one, small, mone), (one, mone, small)):
        x = [_raw(dtype, [b]) for b in order]
        s, a = oracle.direct_sum_f64(x)
        assert s[0] == tiny and a[0] == 2.0 + tiny


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_direct_sum_within_the_summation_bound(dtype):
    """Random patterns over the whole finite range, 16 ranks: within the
    recursive-summation bound (R-1) 2^-53 sum|x| of math.fsum (whose result is
    the correctly rounded sum), for the sum and the magnitude sum."""
    rng = np.random.default_rng(3)
    R, count = 16, 2000
    nbits = 32 if dtype == "fp32" else 16
    x = []
    for _ in range(R):
        bits = rng.integers(0, 1 << nbits, size=count, dtype=np.uint64)
        v = _raw(dtype, bits)
        f = v.astype(np.float64) if dtype != "bf16" else \
            (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ok = np.isfinite(f)
        bits = np.where(ok, bits, 0)
        x.append(_raw(dtype, bits))
    s, a = oracle.direct_sum_f64(x)
    raw = [v.view(np.uint16) if dtype != "fp32" else v.view(np.uint32) for v in x]
    gamma = (R - 1) * 2.0 ** -53
    for i in range(count):
        vals = [_as_float(_decode_exact(raw[r][i], dtype)) for r in range(R)]
        fs = math.fsum(vals)
        fa = math.fsum(abs(v) for v in vals)
        if math.isinf(fs) or math.isinf(fa):
            continue
        assert abs(s[i] - fs) <= gamma * fa * (1 + 1e-12), (i, s[i], fs)
        assert abs(a[i] - fa) <= gamma * fa * (1 + 1e-12)


def test_direct_sum_special_values():
    """An infinity makes the sum infinite, opposite infinities or a NaN make it
    NaN; the magnitude sum is infinite in every case but NaN."""
    inf, ninf, nan, one = 0x7F800000, 0xFF800000, 0x7FC00000, 0x3F800000
    cols = [(inf, one), (inf, ninf), (nan, one), (ninf, ninf)]
    x = [_raw("fp32", [c[r] for c in cols]) for r in range(2)]
    s, a = oracle.direct_sum_f64(x)
    assert s[0] == np.inf and np.isnan(s[1]) and np.isnan(s[2]) and s[3] == -np.inf
    assert a[0] == np.inf and a[1] == np.inf and np.isnan(a[2]) and a[3] == np.inf
