"""CPU oracle for the ring AllReduce -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and shares
no code with it.

The arithmetic lives in ``ring_oracle.c`` (a plain single-threaded ring
simulator); this module loads it with ctypes and adds numpy-facing wrappers plus
the primitive labels of one ring loop derived from the recorded hops.

Arrays: int32 -> ``np.int32``, fp32 -> ``np.float32``, bf16 -> ``np.uint16``
holding the raw bfloat16 bit patterns, fp16 -> ``np.float16``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ring_oracle.c")
_LIB = os.path.join(_HERE, "libring_oracle.so")

DTYPES = {"int32": 0, "fp32": 1, "bf16": 2, "fp16": 3}
NP_DTYPES = {"int32": np.int32, "fp32": np.float32, "bf16": np.uint16, "fp16": np.float16}
OPS = {"sum": 0, "max": 1, "min": 2, "prod": 3}
PRIMITIVES = ["send", "recvReduceSend", "recvReduceCopySend", "recvCopySend", "recv",
              "recvReduceCopy", "copySend"]
MAX_RANKS = 64

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile ring_oracle.c with gcc into oracle/libring_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Hop(ctypes.Structure):
    _fields_ = [("phase", ctypes.c_int32), ("round", ctypes.c_int32), ("hop", ctypes.c_int32),
                ("src", ctypes.c_int32), ("dst", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("bytes", ctypes.c_uint64), ("nterms", ctypes.c_int32),
                ("terms", ctypes.c_uint8 * MAX_RANKS)]


class _Step(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("rank", ctypes.c_int32), ("prim", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("bytes_read", ctypes.c_uint64),
                ("bytes_written", ctypes.c_uint64)]


class _StepLog(ctypes.Structure):
    _fields_ = [("steps", ctypes.POINTER(_Step)), ("capacity", ctypes.c_int32),
                ("used", ctypes.c_int32)]


class _Trace(ctypes.Structure):
    _fields_ = [("hops", ctypes.POINTER(_Hop)), ("capacity", ctypes.c_int32),
                ("used", ctypes.c_int32)]


def _bind(lib):
    vp, u64, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int
    lib.ro_chunk_bounds.argtypes = [u64, i32, i32, ctypes.POINTER(ctypes.c_uint64)]
    lib.ro_allreduce.argtypes = [ctypes.POINTER(vp), i32, u64, i32, i32, ctypes.POINTER(_Trace)]
    lib.ro_reduce_scatter.argtypes = lib.ro_allreduce.argtypes
    lib.ro_all_gather.argtypes = [ctypes.POINTER(vp), i32, u64, i32, ctypes.POINTER(_Trace)]
    lib.ro_allreduce_at.argtypes = [vp, vp, u64, i32, i32, i32, vp]
    lib.ro_direct_sum_f64.argtypes = [ctypes.POINTER(vp), i32, u64, i32, vp, vp]
    lib.ro_staged_allreduce.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, u64, i32, i32,
                                        ctypes.POINTER(_StepLog)]
    lib.ro_reduce_scatter_nccl.argtypes = lib.ro_staged_allreduce.argtypes
    lib.ro_all_gather_nccl.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, u64, i32,
                                       ctypes.POINTER(_StepLog)]
    lib.ro_alltoall.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, u64, i32]
    lib.ro_alltoall.restype = ctypes.c_int
    for f in (lib.ro_chunk_bounds, lib.ro_allreduce, lib.ro_reduce_scatter, lib.ro_all_gather,
              lib.ro_allreduce_at, lib.ro_direct_sum_f64, lib.ro_staged_allreduce,
              lib.ro_reduce_scatter_nccl, lib.ro_all_gather_nccl):
        f.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()  # rebuilds only when the source is newer than the library
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def use_library(path):
    """Point the wrappers at another build of ring_oracle.c (mutation tests).

    Returns the handle in use before, for ``restore_library``.
    """
    global _lib
    prev = _load()
    lib = _bind(ctypes.CDLL(path))
    with _lock:
        _lib = lib
    return prev


def restore_library(handle) -> None:
    global _lib
    with _lock:
        _lib = handle


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _dtype_of(bufs) -> str:
    for name, t in NP_DTYPES.items():
        if bufs[0].dtype == t:
            return name
    raise TypeError(f"unsupported array dtype {bufs[0].dtype}")


def _ptrs(bufs):
    n = bufs[0].size
    for b in bufs:
        if not b.flags.c_contiguous or b.dtype != bufs[0].dtype or b.size != n:
            raise ValueError("rank buffers must be contiguous, same dtype, same length")
    return (ctypes.c_void_p * len(bufs))(*[b.ctypes.data for b in bufs]), n


def chunk_bounds(count: int, R: int, dtype: str) -> np.ndarray:
    """Start of each chunk and the end of the last: R + 1 element offsets."""
    out = (ctypes.c_uint64 * (R + 1))()
    _check(_load().ro_chunk_bounds(count, R, DTYPES[dtype], out), "chunk_bounds")
    return np.array(list(out), dtype=np.uint64)


@dataclass
class Hop:
    phase: str   # "RS" or "AG"
    round: int
    hop: int
    src: int
    dst: int
    chunk: int
    bytes: int
    terms: tuple  # ranks folded into the receiver's chunk, in order


def _run(fn, bufs, dtype_args, trace: bool):
    arr, n = _ptrs(bufs)
    R = len(bufs)
    tr = None
    if trace:
        cap = 2 * R * R
        hops = (_Hop * cap)()
        tr = _Trace(ctypes.cast(hops, ctypes.POINTER(_Hop)), cap, 0)
    rc = fn(arr, R, n, *dtype_args, ctypes.byref(tr) if tr is not None else None)
    _check(rc, fn.__name__)
    if not trace:
        return None
    out = []
    for k in range(min(tr.used, tr.capacity)):
        h = tr.hops[k]
        out.append(Hop("RS" if h.phase == 0 else "AG", h.round, h.hop, h.src, h.dst, h.chunk,
                       int(h.bytes), tuple(h.terms[i] for i in range(h.nterms))))
    return out


def allreduce(bufs, op: str = "sum", trace: bool = False):
    """In-place ring AllReduce of a list of R equal-length numpy arrays."""
    dt = _dtype_of(bufs)
    return _run(_load().ro_allreduce, bufs, (DTYPES[dt], OPS[op]), trace)


def reduce_scatter(bufs, op: str = "sum", trace: bool = False):
    """In-place ring ReduceScatter; afterwards rank r owns chunk (r + 1) mod R."""
    dt = _dtype_of(bufs)
    return _run(_load().ro_reduce_scatter, bufs, (DTYPES[dt], OPS[op]), trace)


def all_gather(bufs, trace: bool = False):
    """In-place ring AllGather of chunk (r + 1) mod R of every rank r."""
    dt = _dtype_of(bufs)
    return _run(_load().ro_all_gather, bufs, (DTYPES[dt],), trace)


def allreduce_at(vals: np.ndarray, chunks: np.ndarray, dtype: str, op: str = "sum") -> np.ndarray:
    """AllReduce result at single positions.

    ``vals`` has shape (npos, R): the R ranks' inputs at each position; ``chunks``
    gives the chunk each position lies in.  Returns an (npos, R) array with every
    rank's result at each position.
    """
    vals = np.ascontiguousarray(vals, dtype=NP_DTYPES[dtype])
    chunks = np.ascontiguousarray(chunks, dtype=np.int32)
    npos, R = vals.shape
    out = np.empty_like(vals)
    rc = _load().ro_allreduce_at(vals.ctypes.data, chunks.ctypes.data, npos, R, DTYPES[dtype],
                                 OPS[op], out.ctypes.data)
    _check(rc, "allreduce_at")
    return out


def direct_sum_f64(bufs):
    """fp64 sum over ranks and fp64 sum of magnitudes, per element."""
    dt = _dtype_of(bufs)
    arr, n = _ptrs(bufs)
    s = np.empty(n, dtype=np.float64)
    a = np.empty(n, dtype=np.float64)
    _check(_load().ro_direct_sum_f64(arr, len(bufs), n, DTYPES[dt], s.ctypes.data,
                                     a.ctypes.data), "direct_sum_f64")
    return s, a


def primitive_labels(hops, R: int):
    """Per-rank primitive sequence of one ring loop, derived from the hops.

    Step k of a rank receives at hop k (k >= 1) and sends at hop k + 1
    (k + 1 <= 2(R - 1)).  A receive in ReduceScatter reduces.  When the chunk in
    hand is finished (it folds all R ranks) and is also sent on, the step keeps
    a copy in the rank's own output as well; a final receive with nothing to
    send just lands the chunk.
    """
    nhops = max(h.hop for h in hops)
    labels = {}
    for rank in range(R):
        seq = []
        for k in range(0, nhops + 1):
            recv = [h for h in hops if h.hop == k and h.dst == rank]
            send = [h for h in hops if h.hop == k + 1 and h.src == rank]
            if not recv:
                seq.append("send" if send else "")
                continue
            h = recv[0]
            name = "recv"
            if h.phase == "RS":
                name += "Reduce"
            if send:
                if len(h.terms) == R:
                    name += "Copy"
                name += "Send"
            seq.append(name)
        labels[rank] = seq
    return labels


@dataclass
class Step:
    step: int
    rank: int
    prim: str
    chunk: int
    bytes_read: int
    bytes_written: int


def _staged(fn, send, recv, n, args, log: bool):
    R = len(send)
    sp = (ctypes.c_void_p * R)(*[b.ctypes.data for b in send])
    rp = (ctypes.c_void_p * R)(*[b.ctypes.data for b in recv])
    lg = None
    if log:
        cap = 2 * R * R
        steps = (_Step * cap)()
        lg = _StepLog(ctypes.cast(steps, ctypes.POINTER(_Step)), cap, 0)
    _check(fn(sp, rp, R, n, *args, ctypes.byref(lg) if lg is not None else None), fn.__name__)
    if not log:
        return None
    return [Step(s.step, s.rank, PRIMITIVES[s.prim], s.chunk, int(s.bytes_read),
                 int(s.bytes_written)) for s in (lg.steps[k] for k in range(min(lg.used, lg.capacity)))]


def _contig(bufs, n, dtype):
    for b in bufs:
        if not b.flags.c_contiguous or b.dtype != NP_DTYPES[dtype] or b.size != n:
            raise ValueError("buffers must be contiguous arrays of the right dtype and length")


def staged_allreduce(send, op: str = "sum", recv=None, log: bool = False):
    """The staged loop of Table V, out of place.  Returns (recv, steps)."""
    dt = _dtype_of(send)
    n = send[0].size
    _contig(send, n, dt)
    if recv is None:
        recv = [np.zeros_like(b) for b in send]
    _contig(recv, n, dt)
    steps = _staged(_load().ro_staged_allreduce, send, recv, n, (DTYPES[dt], OPS[op]), log)
    return recv, steps


def reduce_scatter_nccl(send, op: str = "sum", log: bool = False):
    """send[r] holds R blocks; returns (recv, steps), recv[r] = block r reduced."""
    dt = _dtype_of(send)
    R = len(send)
    total = send[0].size
    if total % R:
        raise ValueError("send buffers must hold R equal blocks")
    _contig(send, total, dt)
    n = total // R
    recv = [np.zeros(n, dtype=NP_DTYPES[dt]) for _ in range(R)]
    steps = _staged(_load().ro_reduce_scatter_nccl, send, recv, n, (DTYPES[dt], OPS[op]), log)
    return recv, steps


def all_gather_nccl(send, log: bool = False):
    """send[r] holds one block; returns (recv, steps), recv[r] = all R blocks."""
    dt = _dtype_of(send)
    R = len(send)
    n = send[0].size
    _contig(send, n, dt)
    recv = [np.zeros(R * n, dtype=NP_DTYPES[dt]) for _ in range(R)]
    steps = _staged(_load().ro_all_gather_nccl, send, recv, n, (DTYPES[dt],), log)
    return recv, steps


def alltoall(send):
    """send[r] holds R blocks; returns recv with recv[q] block r = send[r] block q."""
    R = len(send)
    total = send[0].size
    if total % R:
        raise ValueError("send buffers must hold R equal blocks")
    for b in send:
        if not b.flags.c_contiguous or b.dtype != send[0].dtype or b.size != total:
            raise ValueError("send buffers must be contiguous, same dtype, same length")
    recv = [np.empty_like(send[0]) for _ in range(R)]
    sp = (ctypes.c_void_p * R)(*[b.ctypes.data for b in send])
    rp = (ctypes.c_void_p * R)(*[b.ctypes.data for b in recv])
    _check(_load().ro_alltoall(sp, rp, R, total // R, send[0].itemsize), "alltoall")
    return recv
