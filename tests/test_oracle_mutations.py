"""Plant plausible mistakes in a copy of the CPU oracle and check the pins catch them.

Each mutant is ring_oracle.c with one small edit, built with gcc into a temporary
directory and swapped in through ``oracle.use_library``.  The pins of
test_oracle_pins.py are then run against it; at least one must fail.  The
unmodified source must pass the same pins.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_ops as ops
from tests import test_oracle_pins as pins
from tests import test_oracle_staged as staged

SRC = os.path.join(os.path.dirname(oracle.__file__), "ring_oracle.c")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# (name, text to replace, replacement, which occurrence (0-based))
MUTANTS = [
    ("rs_chunk_index", "int c = mod(r - s + 1, R);", "int c = mod(r + s - 1, R);", 0),
    ("ag_chunk_index", "int c = mod(r + 2 - t, R);", "int c = mod(r + 1 - t, R);", 0),
    ("rs_drops_last_round", "for (int s = 1; s <= R - 1; ++s)", "for (int s = 1; s < R - 1; ++s)", 0),
    ("ag_drops_last_round", "for (int t = 1; t <= R - 1; ++t)", "for (int t = 1; t < R - 1; ++t)", 0),
    ("rs_wrong_receiver", "int q = (r + 1) % R;\n            uint64_t lo = begin[c], n = begin[c + 1] - begin[c];\n            fold_range",
     "int q = (r + R - 1) % R;\n            uint64_t lo = begin[c], n = begin[c + 1] - begin[c];\n            fold_range", 0),
    ("partition_unaligned", "uint64_t chunk_len = (share + per_vector - 1u) / per_vector * per_vector;",
     "uint64_t chunk_len = share;", 0),
    ("partition_floor", "uint64_t share = (count + (uint64_t)R - 1u) / (uint64_t)R;",
     "uint64_t share = count / (uint64_t)R + 1u;", 0),
    ("int_sum_subtracts", "(uint32_t)in[i] + (uint32_t)lo[i]", "(uint32_t)lo[i] - (uint32_t)in[i]", 0),
    ("int_max_is_min", "lo[i] = lo[i] > in[i] ? lo[i] : in[i];", "lo[i] = lo[i] > in[i] ? in[i] : lo[i];", 0),
    ("fp32_max_is_min", "lo[i] = lo[i] > in[i] ? lo[i] : in[i];", "lo[i] = lo[i] > in[i] ? in[i] : lo[i];", 1),
    ("fp32_sum_doubles_local", "lo[i] = in[i] + lo[i];", "lo[i] = in[i] + lo[i] + lo[i] * 0x1p-23f;", 0),
    ("bf16_truncates", "double n = nearbyint(ldexp(a, -q));", "double n = floor(ldexp(a, -q));", 0),
    ("bf16_ties_away", "double n = nearbyint(ldexp(a, -q));", "double n = round(ldexp(a, -q));", 0),
    ("bf16_flushes_subnormals", "if (q < -133) q = -133;", "if (q < -126) q = -126;", 0),
    ("bf16_keeps_9_bits", "int q = e - 8;", "int q = e - 9;", 0),
    ("bf16_overflow_early", "if (r >= 0x1p128)", "if (r >= 0x1p127)", 0),
    ("bf16_max_is_min", "lo[i] = b > a ? lo[i] : in[i];", "lo[i] = b > a ? in[i] : lo[i];", 1),
    ("fp16_max_is_min", "lo[i] = b > a ? lo[i] : in[i];", "lo[i] = b > a ? in[i] : lo[i];", 0),
    ("fp16_truncates", "double r = ldexp(nearbyint(ldexp(a, -q)), q);",
     "double r = ldexp(floor(ldexp(a, -q)), q);", 0),
    ("fp16_flushes_subnormals", "if (q < -24) q = -24;", "if (q < -14) q = -14;", 0),
    ("fp16_overflow_early", "if (r > 65504.0)", "if (r >= 65504.0)", 0),
    ("fp16_keeps_12_bits", "int q = e - 11;", "int q = e - 12;", 0),
    ("fp16_nan_payload", "if (isnan(x)) return 0x7E00u;", "if (isnan(x)) return 0x7E01u;", 0),
    ("int_min_is_max", "lo[i] = lo[i] < in[i] ? lo[i] : in[i];", "lo[i] = lo[i] < in[i] ? in[i] : lo[i];", 0),
    ("fp32_min_is_max", "lo[i] = lo[i] < in[i] ? lo[i] : in[i];", "lo[i] = lo[i] < in[i] ? in[i] : lo[i];", 1),
    ("fp16_min_is_max", "lo[i] = b < a ? lo[i] : in[i];", "lo[i] = b < a ? in[i] : lo[i];", 0),
    ("bf16_min_is_max", "lo[i] = b < a ? lo[i] : in[i];", "lo[i] = b < a ? in[i] : lo[i];", 1),
    ("int_prod_adds", "(uint32_t)in[i] * (uint32_t)lo[i]", "(uint32_t)in[i] + (uint32_t)lo[i]", 0),
    ("fp32_prod_squares", "lo[i] = in[i] * lo[i];", "lo[i] = lo[i] * lo[i];", 0),
    ("fp16_prod_is_sum", "lo[i] = fp16_from_double(a * b);", "lo[i] = fp16_from_double(a + b);", 0),
    ("bf16_prod_truncates", "lo[i] = bf16_from_double(a * b);", "lo[i] = bf16_from_double(a * b * 0x1.0000001p0);", 0),
    ("staged_reads_wrong_slot", "(size_t)((k + 1) & 1)", "(size_t)(k & 1)", 0),
    ("staged_chunk_schedule", "int c = mod(r - k - (mode == STAGED_RS ? 1 : 0), R);",
     "int c = mod(r + k - (mode == STAGED_RS ? 1 : 0), R);", 0),
    ("rs_nccl_unshifted", "(mode == STAGED_RS ? 1 : 0)", "(mode == STAGED_RS ? 0 : 0)", 0),
    ("staged_copy_late", "has_out = k >= R - 1;", "has_out = k >= R;", 0),
    ("staged_reduces_in_allgather", "reduce = k >= 1 && k <= R - 1;", "reduce = k >= 1;", 0),
    ("ag_nccl_skips_own_block", "has_out = 1;", "has_out = k >= 1;", 0),
    ("bf16_nan_payload", "if (isnan(x)) return 0x7FC0u;", "if (isnan(x)) return 0x7FC1u;", 0),
    ("direct_sum_float_accumulator", "double s = 0.0, a = 0.0;", "float s = 0.0f, a = 0.0f;", 0),
    ("direct_sum_abs_without_fabs", "a += fabs(x);", "a += x;", 0),
    ("direct_sum_decodes_bf16_as_fp16", ": dt == RO_BF16 ?", ": dt == RO_FP16 ?", 0),
    ("direct_sum_drops_a_rank", "for (int r = 0; r < R; ++r) {\n            double x", "for (int r = 1; r < R; ++r) {\n            double x", 0),
    ("fp16_decode_subnormal_scale", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);", 0),
    ("ag_reduces", "memcpy((char *)bufs[q] + lo * es, (const char *)bufs[r] + lo * es, n * es);",
     "fold_range(dt, RO_MAX, (const char *)bufs[r] + lo * es, (char *)bufs[q] + lo * es, n);", 0),
]


def _pin_suite():
    """Fast pins; each is a zero-argument callable that raises on failure."""
    return [
        lambda: pins.test_worked_example_schedule(GOLDEN),
        pins.test_worked_example_values,
        lambda: pins.test_table_v_k4(GOLDEN),
        lambda: pins.test_volume_per_rank(7, 7 * 12),
        lambda: pins.test_onehot_tracer(8),
        lambda: pins.test_rank_index_closed_form(8),
        lambda: pins.test_max_of_rank("int32"),
        lambda: pins.test_max_of_rank("fp32"),
        lambda: pins.test_max_of_rank("bf16"),
        lambda: pins.test_brute_force_tiny("fp32", "sum", 5, 37),
        lambda: pins.test_brute_force_tiny("bf16", "sum", 4, 64),
        lambda: pins.test_brute_force_tiny("fp32", "max", 5, 37),
        lambda: pins.test_brute_force_tiny("bf16", "max", 4, 64),
        lambda: pins.test_brute_force_tiny("int32", "sum", 6, 3),
        pins.test_fold_order_is_the_rings,
        pins.test_bf16_add_is_correctly_rounded,
        pins.test_bf16_special_values,
        lambda: pins.test_all_gather_is_a_bit_copy("fp32", 5),
        lambda: pins.test_reduce_scatter_then_all_gather("fp32", "sum", 3),
        pins.test_reduce_scatter_partials,
        lambda: pins.test_direct_sum_decodes_every_16bit_pattern("bf16"),
        lambda: pins.test_direct_sum_decodes_every_16bit_pattern("fp16"),
        pins.test_direct_sum_decodes_fp32_patterns,
        lambda: pins.test_direct_sum_is_the_exact_sum("fp32", "uniform_pm1", 3),
        lambda: pins.test_direct_sum_keeps_far_apart_terms("fp32", 0x30800000),
        lambda: pins.test_direct_sum_keeps_far_apart_terms("fp16", 0x0001),
        pins.test_direct_sum_special_values,
        lambda: pins.test_partition(10, 4, "fp32"),
        lambda: pins.test_partition(100, 8, "bf16"),
        pins.test_edge_cases,
        pins.test_int32_wraps,
        lambda: ops.test_min_prod_brute_force("int32", "min", 5, 37),
        lambda: ops.test_min_prod_brute_force("fp32", "min", 5, 37),
        lambda: ops.test_min_prod_brute_force("bf16", "min", 5, 37),
        lambda: ops.test_min_prod_brute_force("fp16", "min", 5, 37),
        lambda: ops.test_min_prod_brute_force("int32", "prod", 5, 37),
        lambda: ops.test_min_prod_brute_force("fp32", "prod", 5, 37),
        lambda: ops.test_min_prod_brute_force("bf16", "prod", 5, 37),
        lambda: ops.test_min_prod_brute_force("fp16", "prod", 5, 37),
        lambda: ops.test_fp16_sum_max_brute_force("sum", 4, 64),
        lambda: ops.test_fp16_sum_max_brute_force("max", 4, 64),
        lambda: ops.test_fp16_hop_is_correctly_rounded("sum", 3000),
        lambda: ops.test_fp16_hop_is_correctly_rounded("prod", 3000),
        ops.test_fp16_special_values,
        lambda: ops.test_bf16_product_is_correctly_rounded(3000),
        lambda: staged.test_staged_primitives_table_v_k4(GOLDEN),
        lambda: staged.test_staged_chunks_follow_the_worked_example(GOLDEN),
        lambda: staged.test_staged_traffic("fp32", 5, 37 * 5 + 3),
        lambda: staged.test_staged_allreduce_brute_force("fp32", "sum", 5, 37),
        lambda: staged.test_staged_allreduce_brute_force("int32", "max", 4, 64),
        lambda: staged.test_reduce_scatter_nccl_brute_force("fp32", "sum", 5, 4),
        lambda: staged.test_all_gather_nccl_is_the_gather("fp16", 5, 17),
        lambda: staged.test_all_gather_nccl_is_the_gather("int32", 3, 5),
    ]


def _build(src_text, workdir, name):
    c_path = os.path.join(workdir, name + ".c")
    so_path = os.path.join(workdir, name + ".so")
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-w",
                    "-o", so_path, c_path, "-lm"], check=True)
    return so_path


def _failures(so_path, first_only=False):
    """Indices of the pins that fail against the library at so_path (only the
    first one with first_only)."""
    prev = oracle.use_library(so_path)
    failed = []
    try:
        for k, pin in enumerate(_pin_suite()):
            try:
                pin()
            except (AssertionError, ValueError):
                failed.append(k)
                if first_only:
                    break
    finally:
        oracle.restore_library(prev)
    return failed


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def _mutate(text, old, new, occurrence):
    pos = -1
    for _ in range(occurrence + 1):
        pos = text.find(old, pos + 1)
        assert pos >= 0, f"mutation anchor not found: {old!r}"
    return text[:pos] + new + text[pos + len(old):]


def test_unmutated_oracle_passes_the_suite(workdir):
    with open(SRC) as f:
        text = f.read()
    assert _failures(_build(text, workdir, "original")) == []


@pytest.mark.parametrize("name,old,new,occurrence", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, old, new, occurrence):
    with open(SRC) as f:
        text = f.read()
    so = _build(_mutate(text, old, new, occurrence), workdir, name)
    assert _failures(so, first_only=True), f"no pin caught mutant {name}"
