"""Seeded synthetic inputs for the ring AllReduce workloads.

This module only draws input arrays: it holds none of the collective's
arithmetic and is shared by the tests, the benchmark and the smoke check so
that the GPU library and the CPU oracle see the same bits.

Every rank r draws from its own numpy PCG64 stream seeded ``seed*1000 + r``.
Arrays: int32 -> ``np.int32``, fp32 -> ``np.float32``, bf16 -> ``np.uint16``
(raw bfloat16 bits; the fp32 draw is converted by torch's round-to-nearest-even
cast).

Workloads (sizes are per rank):

* ``worked_example`` -- the 4-GPU example of the post "Why AllReduce =
  ReduceScatter + AllGather -- with NCCL Ring AllReduce" (sections 1 and 5):
  R=4, 4 chunks of 16 int32, integers uniform in [-1000, 1000], SUM, 1 slice.
* ``r8_fp32_64MiB`` -- R=8, fp32, 64 MiB, uniform in [-1, 1), SUM, 4 slices.
* ``r8_bf16_256MiB`` -- R=8, bf16, 256 MiB, normal(0, 1), SUM, 8 slices.
* ``r16_fp32_sweep`` -- R=16, fp32, 4 KiB * 4^k for k = 0..9 (4 KiB .. 1 GiB),
  uniform in [-1, 1), SUM and MAX, 1..16 slices, counting-barrier step sync.
* ``r16_fp32_1GiB`` -- the largest point of that sweep as a workload of its own:
  R=16, fp32, 1 GiB, uniform in [-1, 1), SUM, 16 slices, counting-barrier step
  sync (the same inputs as sweep point k = 9).
* ``r64_fp32_32MiB`` -- R=64, fp32, 32 MiB, uniform in [-1, 1), SUM, 8 slices
  as independent contexts, counting-barrier step sync (R-1 arrivals per step).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

NP_DTYPES = {"int32": np.int32, "fp32": np.float32, "bf16": np.uint16, "fp16": np.float16}
ELEM_BYTES = {"int32": 4, "fp32": 4, "bf16": 2, "fp16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    R: int
    dtype: str
    op: str
    count: int          # elements per rank
    nslices: int
    seed: int
    dist: str
    sync: str = "p2p"   # "p2p" (predecessor hand-off) or "barrier" (all ranks per step)

    @property
    def bytes_per_rank(self) -> int:
        return self.count * ELEM_BYTES[self.dtype]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


KiB = 1024
MiB = 1024 * KiB

WORKED_EXAMPLE = Workload("worked_example", 4, "int32", "sum", 64, 1, 1, "int_pm1000")
R8_FP32_64MIB = Workload("r8_fp32_64MiB", 8, "fp32", "sum", 64 * MiB // 4, 4, 2, "uniform_pm1")
R8_BF16_256MIB = Workload("r8_bf16_256MiB", 8, "bf16", "sum", 256 * MiB // 2, 8, 3, "normal")
R64_FP32_32MIB = Workload("r64_fp32_32MiB", 64, "fp32", "sum", 32 * MiB // 4, 8, 5,
                          "uniform_pm1", sync="barrier")


def r16_sweep(k: int, op: str = "sum", nslices: int = 4) -> Workload:
    """R=16 fp32 sweep point k: 4 KiB * 4^k per rank (k = 0 .. 9)."""
    if not 0 <= k <= 9:
        raise ValueError("sweep index k must be in 0..9")
    count = (4 * KiB * 4 ** k) // 4
    return Workload(f"r16_fp32_{4 * 4 ** k}KiB_{op}_ns{nslices}", 16, "fp32", op, count,
                    nslices, 40 + k, "uniform_pm1", sync="barrier")


R16_FP32_1GIB = r16_sweep(9, "sum", 16).with_(name="r16_fp32_1GiB")

ALL = {w.name: w for w in (WORKED_EXAMPLE, R8_FP32_64MIB, R8_BF16_256MIB, R64_FP32_32MIB,
                           R16_FP32_1GIB)}


def _draw(dist: str, dtype: str, count: int, rank: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed * 1000 + rank)
    if dist == "int_pm1000":
        x = rng.integers(-1000, 1001, size=count, dtype=np.int32)
    elif dist == "uniform_pm1":
        x = rng.random(count, dtype=np.float32)
        x *= 2.0
        x -= 1.0
    elif dist == "normal":
        x = rng.standard_normal(count, dtype=np.float32)
    elif dist == "unit_jitter":      # magnitudes in [7/8, 9/8), random sign: long products stay finite
        x = rng.random(count, dtype=np.float32)
        x = (x - np.float32(0.5)) * np.float32(0.25) + np.float32(1.0)
        x *= np.where(rng.random(count) < 0.5, np.float32(-1.0), np.float32(1.0)).astype(np.float32)
        if dtype == "int32":
            x = rng.integers(-3, 4, size=count, dtype=np.int32)
    elif dist == "onehot":           # rank r contributes the single bit 1 << r
        x = np.full(count, 1 << rank, dtype=np.int64)
    elif dist == "rank_index":       # rank r, position i holds r*1000 + i
        x = rank * 1000 + np.arange(count, dtype=np.int64)
    elif dist == "rank":             # rank r holds r everywhere
        x = np.full(count, rank, dtype=np.int64)
    elif dist == "bits":             # uniformly random bit patterns (NaN payloads included)
        x = rng.integers(0, 1 << 32, size=count, dtype=np.uint32)
        if dtype == "bf16":
            return (x & 0xFFFF).astype(np.uint16)
        if dtype == "fp16":
            return (x & 0xFFFF).astype(np.uint16).view(np.float16)
        return x.view(NP_DTYPES[dtype])
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return _as_dtype(x, dtype)


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "int32":
        return x.astype(np.int32, copy=False)
    if dtype == "fp32":
        return x.astype(np.float32, copy=False)
    if dtype == "fp16":
        return x.astype(np.float32, copy=False).astype(np.float16)  # round to nearest even
    import torch  # the cast below is torch's round-to-nearest-even conversion
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def generate(R: int, count: int, dtype: str, dist: str, seed: int, threads: int = 8):
    """R seeded arrays of ``count`` elements each."""
    with ThreadPoolExecutor(max_workers=max(1, min(threads, R))) as ex:
        return list(ex.map(lambda r: _draw(dist, dtype, count, r, seed), range(R)))


def inputs(w: Workload, threads: int = 8):
    return generate(w.R, w.count, w.dtype, w.dist, w.seed, threads)
