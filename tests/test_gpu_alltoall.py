"""GPU parity of the AlltoAll (the 2kiu.com article on NCCL GIN, section "a pure
GIN AlltoAll kernel") against the CPU oracle, bit for bit, and of its counting
signal: one per receiver, advanced by every sender's every part."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import RAW_NP, log, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_allreduce_amd
    ring_allreduce_amd.init()
    return ring_allreduce_amd


def _check(rr, x, dtype, **opts):
    send = [to_device(a, dtype) for a in x]
    recv = rr.alltoall(send, None, **opts)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    want = oracle.alltoall(x)
    for q in range(len(x)):
        got = to_host(recv[q], dtype)
        assert np.array_equal(got, want[q].view(RAW_NP[dtype])), f"receiver {q}"
    for a, t in zip(x, send):
        assert np.array_equal(to_host(t, dtype), a.view(RAW_NP[dtype]))


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16", "fp16"])
@pytest.mark.parametrize("R,n", [(1, 7), (2, 5), (3, 64), (5, 1001), (8, 4096), (8, 4099),
                                 (16, 333), (64, 257)])
def test_alltoall_matches_oracle(rr, dtype, R, n):
    log(f"case alltoall {dtype} R={R} n={n}")
    _check(rr, workloads.generate(R, R * n, dtype, "bits", 100 + R), dtype)


def test_alltoall_gin_sample_pattern(rr):
    """The article's check: rank r's block for rank d holds r*1000 + d*100 + i."""
    R, n = 8, 1000
    i = np.arange(n, dtype=np.int64)
    x = [np.concatenate([r * 1000 + d * 100 + i for d in range(R)]).astype(np.int32)
         for r in range(R)]
    send = [to_device(a, "int32") for a in x]
    recv = rr.alltoall(send)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    for d in range(R):
        got = recv[d].cpu().numpy()
        for r in range(R):
            assert np.array_equal(got[r * n:(r + 1) * n], (r * 1000 + d * 100 + i).astype(np.int32))


def test_alltoall_repeated_calls_and_plan(rr):
    """The receivers' shadows advance by R * parts per call, so back-to-back
    calls need no reset; the plan gives the parts and the traffic."""
    R, n = 8, (1 << 18) + 3
    p = rr.plan(R, n, "fp32", 1, phase="alltoall")
    assert p["hbm_bytes"] == 2 * R * R * n * 4 and p["grid"] == R * p["team"]
    x = workloads.generate(R, R * n, "fp32", "bits", 7)
    for k in range(4):
        log(f"case alltoall repeat {k}")
        _check(rr, x, "fp32")


@pytest.mark.parametrize("inject", ["extra", "drop"])
def test_alltoall_timeout_and_recovery(rr, inject):
    R, n = 4, 4096
    x = workloads.generate(R, R * n, "int32", "bits", 8)
    send = [to_device(a, "int32") for a in x]
    flag = rr.INJECT_EXTRA_EXPECTED if inject == "extra" else rr.INJECT_DROP_ARRIVAL
    log(f"case alltoall timeout {inject}")
    rr.alltoall(send, None, inject=flag, timeout_ns=20_000_000)
    st, rec = rr.last_kernel_error()
    assert st == rr.RR_ERR_TIMEOUT and rec["expected"] - rec["observed"] == 1
    if inject == "extra":
        assert rec["waiter"] == 0
    _check(rr, x, "int32")


def test_alltoall_full_size(rr):
    w = workloads.R8_FP32_64MIB
    log("case alltoall full size")
    x = workloads.inputs(w)
    _check(rr, x, "fp32")
