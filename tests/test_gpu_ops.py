"""GPU parity of the in-place ring for fp16 and for MIN and PROD: the HIP kernels
against the CPU oracle, element by element, bit for bit."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import assert_matches_oracle, log, oracle_expect, to_host, to_slabs, guards_intact

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
