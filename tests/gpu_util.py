"""Helpers for the GPU parity tests: move seeded host inputs to rank buffers on
the GPU, run the library, compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TORCH = {"int32": torch.int32, "fp32": torch.float32, "bf16": torch.bfloat16,
         "fp16": torch.float16}
RAW_NP = {"int32": np.uint32, "fp32": np.uint32, "bf16": np.uint16, "fp16": np.uint16}
RAW_TORCH = {"int32": torch.int32, "fp32": torch.int32, "bf16": torch.int16, "fp16": torch.int16}
SIGNED_NP = {"int32": np.int32, "fp32": np.int32, "bf16": np.int16, "fp16": np.int16}

GUARD_FILL = {"int32": -0x5A5A5A5B, "fp32": -1.2345e-19, "bf16": -1.2345e-19, "fp16": -1.5e-5}


def log(msg: str) -> None:
    print(msg, flush=True)


def to_slabs(rr, x, dtype, guard=True):
    """Copy host arrays into one device allocation (guard bands between ranks)."""
    R, count = len(x), x[0].size
    slabs = rr.make_slabs(R, count, TORCH[dtype], device="cuda",
                          fill=GUARD_FILL[dtype] if guard else None)
    for r in range(R):
        slabs.ranks[r].view(RAW_TORCH[dtype]).copy_(
            torch.from_numpy(x[r].view(RAW_NP[dtype]).view(SIGNED_NP[dtype])))
    return slabs


def to_device(a, dtype):
    """One host array to a new device tensor, bit for bit."""
    t = torch.empty(a.size, dtype=TORCH[dtype], device="cuda")
    t.view(RAW_TORCH[dtype]).copy_(torch.from_numpy(a.view(RAW_NP[dtype]).view(SIGNED_NP[dtype])))
    return t


def to_host(t, dtype):
    """Raw bits of a device buffer as a numpy array."""
    return t.view(RAW_TORCH[dtype]).cpu().numpy().view(RAW_NP[dtype])


def guards_intact(slabs, dtype, count):
    """Everything outside the R rank buffers still holds the fill pattern."""
    st = slabs.storage
    R = len(slabs.ranks)
    # the gap after each rank buffer (the last one runs to the end of the storage)
    gaps = [(r * slabs.stride + count, (r + 1) * slabs.stride if r + 1 < R else st.numel())
            for r in range(R)]
    for lo, hi in gaps:
        if hi <= lo:
            continue
        piece = st[lo:hi]
        ref = torch.full_like(piece, GUARD_FILL[dtype])
        if not torch.equal(piece.view(RAW_TORCH[dtype]), ref.view(RAW_TORCH[dtype])):
            return False
    return True


def bits_equal(a, b, dtype):
    """Bitwise equality, except that fp32 NaNs compare equal whatever the payload
    (x86 and gfx950 propagate NaN payloads differently; bf16 results are
    canonicalised on both sides)."""
    ra, rb = a.view(RAW_NP[dtype]), b.view(RAW_NP[dtype])
    eq = ra == rb
    if dtype == "fp32":
        fa, fb = a.view(np.float32), b.view(np.float32)
        eq |= np.isnan(fa) & np.isnan(fb)
    return eq


def oracle_expect(x, op, phase="allreduce"):
    e = [a.copy() for a in x]
    if phase == "allreduce":
        oracle.allreduce(e, op)
    elif phase == "reduce_scatter":
        oracle.reduce_scatter(e, op)
    else:
        oracle.all_gather(e)
    return e


def assert_matches_oracle(got, expect, dtype, what=""):
    for r in range(len(expect)):
        eq = bits_equal(got[r], expect[r], dtype)
        if not eq.all():
            bad = np.flatnonzero(~eq)
            k = bad[0]
            raise AssertionError(
                f"{what}: rank {r} differs from the oracle at {bad.size} of {eq.size} elements; "
                f"first at {k}: got {got[r].view(RAW_NP[dtype])[k]:#x} "
                f"want {expect[r].view(RAW_NP[dtype])[k]:#x}")


def sample_positions(count, R, dtype, nslices, plan, n_random, seed):
    """Random positions plus every chunk / slice / team boundary (both sides)."""
    rng = np.random.default_rng(seed)
    pts = set(rng.integers(0, count, size=min(n_random, count)).tolist())
    pts.update([0, count - 1])
    CL, SL, TL = plan["chunk_len"], plan["slice_len"], plan["sub_len"]
    for c in range(R):
        base = c * CL
        for j in range(nslices + 1):
            s0 = base + j * SL
            for p in (s0 - 1, s0, s0 + 1):
                if 0 <= p < count:
                    pts.add(p)
        for k in range(0, max(1, SL // max(TL, 1)) + 1):
            p = base + k * TL
            if 0 <= p < count:
                pts.add(p)
            if 0 <= p - 1 < count:
                pts.add(p - 1)
    return np.array(sorted(pts), dtype=np.int64)


def oracle_at(x, pos, dtype, op):
    """Oracle results at positions ``pos`` for every rank: array (npos, R)."""
    R, count = len(x), x[0].size
    bounds = oracle.chunk_bounds(count, R, dtype).astype(np.int64)
    chunks = np.searchsorted(bounds, pos, side="right") - 1
    vals = np.stack([x[r][pos] for r in range(R)], axis=1)
    return oracle.allreduce_at(vals, chunks, dtype, op)


def assert_full_matches(dev_ranks, expect, dtype, what="", piece=1 << 26):
    """Every element of every rank buffer on the device against the expected host
    arrays, bit for bit (fp32 NaNs compare equal whatever the payload), read back
    one piece of each rank at a time so that host memory stays bounded."""
    for r, (t, e) in enumerate(zip(dev_ranks, expect)):
        want_all = e.view(RAW_NP[dtype])
        assert t.numel() == want_all.size, f"{what}: rank {r} has {t.numel()} elements"
        raw = t.view(RAW_TORCH[dtype])
        for lo in range(0, want_all.size, piece):
            hi = min(lo + piece, want_all.size)
            got = raw[lo:hi].cpu().numpy().view(RAW_NP[dtype])
            want = want_all[lo:hi]
            if np.array_equal(got, want):
                continue
            eq = bits_equal(got, want, dtype)
            if eq.all():
                continue
            bad = np.flatnonzero(~eq)
            k = bad[0]
            raise AssertionError(
                f"{what}: rank {r} differs from the oracle at {bad.size} of {hi - lo} elements "
                f"in [{lo}, {hi}); first at {lo + k}: got {got[k]:#x} want {want[k]:#x}")
