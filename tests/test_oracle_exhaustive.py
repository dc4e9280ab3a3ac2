"""Exhaustive pins of the oracle's 16-bit hop: every one of the 2^32 ordered
pairs (a, b) of bfloat16 or binary16 bit patterns through its SUM and PROD
folds, and a strided sweep of the MAX and MIN selections.

The per-hop fold of the post "Why AllReduce = ReduceScatter + AllGather -- with
NCCL Ring AllReduce" (loosp.cn, section 5: the incoming partial is added to the
local one) is, for a 16-bit format, the exact sum rounded once to the format,
nearest even.  The reference sits in tests/c/exhaustive_hop.c: both operands
decoded by numpy (a table of all 65536 patterns), added in binary64 and rounded
to the format by integer operations on the binary64 bits; a NaN result is the
canonical quiet NaN.  PROD: the binary64 product of the two decoded values
(exact) rounded the same way: the correctly rounded product.  MAX / MIN select the local operand if it compares greater (less)
than the incoming one, else the incoming one.  The reference shares no code
with the oracle, which it calls through dlopen.  About a minute per fold on 8
cores (marked slow); strided runs check that the same harness catches planted
mistakes.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "ring_oracle.c")


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    d = tmp_path_factory.mktemp("exhaustive")
    exe = str(d / "exhaustive_hop")
    build = subprocess.run([gcc, "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pthread",
                            os.path.join(HERE, "c", "exhaustive_hop.c"), "-o", exe, "-ldl", "-lm"],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        tables = _tables(bits)
    paths = {}
    for name, t in tables.items():
        p = d / f"decode_{name}.bin"
        t.astype("<f8").tofile(p)
        paths[name] = str(p)
    return exe, paths, d


def _tables(bits):
    return {
        # bfloat16 is the upper half of a binary32: decode through numpy's float32
        "bf16": (bits << 16).view(np.float32).astype(np.float64),
        # binary16 through numpy's float16
        "fp16": bits.astype(np.uint16).view(np.float16).astype(np.float64),
    }


def _run(harness, lib, dtype, step=1, op="sum"):
    exe, paths, _ = harness
    code = oracle.DTYPES[dtype]
    run = subprocess.run([exe, lib, str(code), paths[dtype], str(_threads()), str(step),
                          str(oracle.OPS[op])],
                         capture_output=True, text=True, timeout=1200)
    assert run.returncode == 0, run.stdout + run.stderr
    first = run.stdout.split()
    pairs, mismatches = int(first[1]), int(first[3])
    return pairs, mismatches, run.stdout


def test_decode_tables_are_the_formats(harness):
    """The tables the reference reads: a few values fixed by the formats."""
    _, paths, _ = harness
    bf = np.fromfile(paths["bf16"], dtype="<f8")
    hf = np.fromfile(paths["fp16"], dtype="<f8")
    assert bf[0x3F80] == 1.0 and bf[0xC000] == -2.0 and bf[0x0001] == 2.0 ** -133
    assert bf[0x7F7F] == (2 - 2 ** -7) * 2.0 ** 127 and np.isinf(bf[0x7F80]) and np.isnan(bf[0x7FC1])
    assert hf[0x3C00] == 1.0 and hf[0x0001] == 2.0 ** -24 and hf[0x7BFF] == 65504.0
    assert np.isinf(hf[0xFC00]) and hf[0xFC00] < 0 and np.isnan(hf[0x7E01])


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_every_pair_through_the_sum_fold(harness, dtype):
    """All 2^32 ordered operand pairs: the oracle's hop equals the reference."""
    lib = oracle.build()
    pairs, mismatches, out = _run(harness, lib, dtype)
    assert pairs == 1 << 32
    assert mismatches == 0, out


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_every_pair_through_the_prod_fold(harness, dtype):
    """All 2^32 ordered operand pairs through the PROD fold."""
    lib = oracle.build()
    pairs, mismatches, out = _run(harness, lib, dtype, op="prod")
    assert pairs == 1 << 32
    assert mismatches == 0, out


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_max_min_selections(harness, dtype, op):
    """Every 61st first operand against all 65536 second ones (70 million pairs,
    every sign, zero, subnormal, infinity and NaN class on both sides)."""
    lib = oracle.build()
    pairs, mismatches, out = _run(harness, lib, dtype, step=61, op=op)
    assert pairs == 1075 * 65536
    assert mismatches == 0, out


@pytest.mark.parametrize("dtype,op,old,new", [
    ("bf16", "sum", "double n = nearbyint(ldexp(a, -q));", "double n = floor(ldexp(a, -q));"),
    ("bf16", "sum", "if (q < -133) q = -133;", "if (q < -126) q = -126;"),
    ("fp16", "sum", "double r = ldexp(nearbyint(ldexp(a, -q)), q);",
     "double r = ldexp(round(ldexp(a, -q)), q);"),
    ("fp16", "sum", "if (r > 65504.0)", "if (r >= 65504.0)"),
    ("bf16", "prod", "lo[i] = bf16_from_double(a * b);", "lo[i] = bf16_from_double(a * a);"),
    ("fp16", "max", "lo[i] = b > a ? lo[i] : in[i];", "lo[i] = b >= a ? lo[i] : in[i];"),
])
def test_the_harness_catches_planted_mistakes(harness, dtype, op, old, new):
    """A strided run (every 257th first operand) against oracles with one
    mistake planted in a fold or its rounding: each is caught, while the
    unmodified oracle passes the same run."""
    _, _, d = harness
    with open(ORACLE_SRC) as f:
        text = f.read()
    assert old in text
    libs = {}
    for tag, src in (("ok", text), ("bad", text.replace(old, new, 1))):
        c = d / f"oracle_{dtype}_{tag}_{abs(hash(new)) % 10 ** 8}.c"
        so = str(c)[:-2] + ".so"
        c.write_text(src)
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-w",
                        "-o", so, str(c), "-lm"], check=True)
        libs[tag] = so
    pairs, mismatches, out = _run(harness, libs["ok"], dtype, step=257, op=op)
    assert pairs == 256 * 65536 and mismatches == 0, out
    _, mismatches, _ = _run(harness, libs["bad"], dtype, step=257, op=op)
    assert mismatches > 0
