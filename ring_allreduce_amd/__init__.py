"""Ring AllReduce over virtual ranks on one MI355X -- Python binding.

A thin ctypes layer over ``librr.so`` (declared in ``include/rr.h``).  It only
marshals arguments: tensors become device pointers, dtype and op names become
enum values, a torch stream becomes a ``hipStream_t``.  Every step of the
collective runs in the library's HIP kernels; there is no fallback.  Importing
this package without a built ``librr.so`` raises.

PyTorch supplies device memory and streams.  ``import torch`` happens first so
that ``librr.so`` binds to the same HIP runtime instance as torch.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # noqa: F401  (loads the HIP runtime librr.so must share)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librr.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
        "or python ring_allreduce_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

RR_MAX_RANKS = 64
RR_MAX_SLICES = 1024

DTYPES = {"int32": 0, "fp32": 1, "bf16": 2, "fp16": 3}
OPS = {"sum": 0, "max": 1, "min": 2, "prod": 3}
SYNCS = {"auto": 0, "p2p": 1, "barrier": 2, "launch": 3, "per_peer": 4}
SYNC_NAMES = {v: k for k, v in SYNCS.items()}
PHASES = {"allreduce": 0, "reduce_scatter": 1, "all_gather": 2, "allreduce_staged": 3,
          "reduce_scatter_blocks": 4, "all_gather_blocks": 5, "alltoall": 6}

STATUS = {0: "RR_OK", 1: "RR_ERR_INVALID", 2: "RR_ERR_UNSUPPORTED", 3: "RR_ERR_HIP",
          4: "RR_ERR_TIMEOUT", 5: "RR_ERR_NOMEM"}
RR_OK, RR_ERR_INVALID, RR_ERR_UNSUPPORTED, RR_ERR_HIP, RR_ERR_TIMEOUT, RR_ERR_NOMEM = range(6)

INJECT_EXTRA_EXPECTED = 0x1
INJECT_DROP_ARRIVAL = 0x2
INJECT_DEFER_ARRIVAL = 0x4
FLAG_NO_XCD_MAP = 0x1
FLAG_NO_POINTER_CHECK = 0x2
FLAG_COOPERATIVE = 0x4
FLAG_FUSED_BOUNDARY = 0x8
FLAG_AUDIT = 0x10
FLAG_STREAM_LOADS = 0x20
FLAG_CACHED_LOADS = 0x40
FLAG_SHARED_SIGNAL = 0x80
FLAG_WAITER_SIGNAL = 0x800
FLAG_POLL_FAST = 0x100
FLAG_POLL_MEDIUM = 0x200
FLAG_POLL_SLOW = 0x400
FLAG_ASCENDING = 0x1000
FLAG_ALTERNATE = 0x2000

_TORCH_DTYPES = {torch.int32: "int32", torch.float32: "fp32", torch.bfloat16: "bf16",
                 torch.float16: "fp16"}
ELEM_BYTES = {"int32": 4, "fp32": 4, "bf16": 2, "fp16": 2}


class Options(ctypes.Structure):
    _fields_ = [("sync", ctypes.c_int32), ("team", ctypes.c_int32), ("block", ctypes.c_int32),
                ("rounds", ctypes.c_int32), ("timeout_ns", ctypes.c_uint64),
                ("inject", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("depth", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [("sync", ctypes.c_int32), ("team", ctypes.c_int32), ("block", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("xcd_map", ctypes.c_int32), ("cooperative", ctypes.c_int32),
                ("resident_max", ctypes.c_int32), ("rounds", ctypes.c_int32),
                ("depth", ctypes.c_int32), ("fused", ctypes.c_int32),
                ("stream_loads", ctypes.c_int32), ("alternate", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("chunk_len", ctypes.c_uint64),
                ("slice_len", ctypes.c_uint64), ("sub_len", ctypes.c_uint64),
                ("hbm_bytes", ctypes.c_uint64)]


class ErrorRecord(ctypes.Structure):
    _fields_ = [("status", ctypes.c_int32), ("ctx", ctypes.c_int32), ("waiter", ctypes.c_int32),
                ("hop", ctypes.c_int32), ("peer", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("expected", ctypes.c_uint64),
                ("observed", ctypes.c_uint64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_u64 = ctypes.c_uint64
_OPT = ctypes.POINTER(Options)


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_allreduce_ring_ex = _sig("allreduce_ring_ex", _i, ctypes.POINTER(_vp), _i, _sz, _i, _i, _i, _OPT, _vp)
_reduce_scatter_ring_ex = _sig("reduce_scatter_ring_ex", _i, ctypes.POINTER(_vp), _i, _sz, _i, _i,
                               _i, _OPT, _vp)
_all_gather_ring_ex = _sig("all_gather_ring_ex", _i, ctypes.POINTER(_vp), _i, _sz, _i, _i, _OPT, _vp)
_allreduce_ring = _sig("allreduce_ring", _i, ctypes.POINTER(_vp), _i, _sz, _i, _i, _i, _vp)
_allreduce_ring_timed = _sig("allreduce_ring_timed", _i, ctypes.POINTER(_vp), _i, _sz, _i, _i, _i,
                             _OPT, _vp, _sz, ctypes.POINTER(ctypes.c_uint32), _vp)
_reduce_scatter_ring = _sig("reduce_scatter_ring", _i, ctypes.POINTER(_vp), _i, _sz, _i, _i, _i, _vp)
_all_gather_ring = _sig("all_gather_ring", _i, ctypes.POINTER(_vp), _i, _sz, _i, _i, _vp)
_plan_query = _sig("rr_plan_query", _i, _i, _sz, _i, _i, _i, _OPT, ctypes.POINTER(_Plan))
_allreduce_ring_staged = _sig("allreduce_ring_staged", _i, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                              _i, _sz, _i, _i, _i, _OPT, _vp)
_allreduce_ring_staged_noalloc = _sig("allreduce_ring_staged_noalloc", _i, ctypes.POINTER(_vp),
                                      ctypes.POINTER(_vp), _i, _sz, _i, _i, _i, _OPT, _vp)
_reduce_scatter = _sig("reduce_scatter", _i, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i, _sz, _i,
                       _i, _i, _OPT, _vp)
_all_gather = _sig("all_gather", _i, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i, _sz, _i, _i,
                   _OPT, _vp)
_alltoall = _sig("alltoall", _i, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i, _sz, _i, _OPT, _vp)
_cb_create = _sig("counting_barrier_create", _i, _i, _i, ctypes.POINTER(_vp))
_cb_destroy = _sig("counting_barrier_destroy", _i, _vp)
_cb_reset = _sig("counting_barrier_reset", _i, _vp, _vp)
_cb_preset = _sig("counting_barrier_preset", _i, _vp, _u64, _vp)
_cb_read = _sig("counting_barrier_read", _i, _vp, _i, _i, ctypes.POINTER(_u64), ctypes.POINTER(_u64))
_cb_read_peer = _sig("counting_barrier_read_peer", _i, _vp, _i, _i, _i, ctypes.POINTER(_u64),
                     ctypes.POINTER(_u64))
_cb_early = _sig("counting_barrier_early_passes", _i, _vp, _i, _i, ctypes.POINTER(_u64))
_cb_run = _sig("counting_barrier_run", _i, _vp, _i, _i, _i, _u64, _OPT, _vp)
_cb_run_timed = _sig("counting_barrier_run_timed", _i, _vp, _i, _i, _i, _u64, _OPT, _vp,
                     ctypes.POINTER(ctypes.c_uint32), _vp)
_last_kernel_error = _sig("rr_last_kernel_error", _i, _vp, ctypes.POINTER(ErrorRecord))
_init = _sig("rr_init", _i)
_workspace_preset = _sig("rr_workspace_preset", _i, _u64, _vp)
_hbm_copy = _sig("rr_hbm_copy", _i, _vp, _vp, _sz, _vp)
_status_string = _sig("rr_status_string", ctypes.c_char_p, _i)
_abi_version = _sig("rr_abi_version", _i)
_finalize = _sig("rr_finalize", None)

# Every symbol include/rr.h declares, for the export check.
EXPORTED = ["allreduce_ring", "reduce_scatter_ring", "all_gather_ring", "allreduce_ring_ex",
            "reduce_scatter_ring_ex", "all_gather_ring_ex", "allreduce_ring_staged",
            "allreduce_ring_staged_noalloc", "allreduce_ring_timed",
            "reduce_scatter", "all_gather", "alltoall", "rr_plan_query",
            "counting_barrier_create", "counting_barrier_destroy", "counting_barrier_reset",
            "counting_barrier_preset", "counting_barrier_read", "counting_barrier_read_peer",
            "counting_barrier_early_passes", "counting_barrier_run", "counting_barrier_run_timed",
            "rr_last_kernel_error", "rr_init", "rr_workspace_preset", "rr_hbm_copy",
            "rr_status_string", "rr_abi_version", "rr_finalize"]


class RRError(RuntimeError):
    def __init__(self, status: int, what: str, record: dict | None = None):
        self.status = status
        self.record = record
        msg = f"{what}: {status_string(status)}"
        if record:
            missing = record["expected"] - record["observed"]
            msg += (f" (context {record['ctx']}, waiter rank {record['waiter']}, hop {record['hop']}: "
                    f"expected signal {record['expected']}, saw {record['observed']}, "
                    f"{missing} arrival(s) missing)")
        super().__init__(msg)


def status_string(status: int) -> str:
    return _status_string(status).decode()


def abi_version() -> int:
    return _abi_version()


def _check(status: int, what: str) -> None:
    if status != RR_OK:
        raise RRError(status, what)


def _stream_handle(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_LOADS = {"auto": 0, "stream": FLAG_STREAM_LOADS, "cached": FLAG_CACHED_LOADS}
_ORDERS = {"auto": 0, "alternate": FLAG_ALTERNATE, "ascending": FLAG_ASCENDING}


def _options(sync="auto", team=0, block=0, rounds=0, timeout_ns=0, inject=0, flags=0, depth=0,
             fused=False, loads="auto", order="auto"):
    if fused:
        flags |= FLAG_FUSED_BOUNDARY
    flags |= _LOADS[loads] | _ORDERS[order]
    return Options(SYNCS[sync] if isinstance(sync, str) else int(sync), team, block, rounds,
                   timeout_ns, inject, flags, depth, 0)


def _buffers(tensors):
    if not tensors:
        raise ValueError("need at least one rank buffer")
    t0 = tensors[0]
    if t0.dtype not in _TORCH_DTYPES:
        raise TypeError(f"unsupported dtype {t0.dtype}; use int32, float32, bfloat16 or float16")
    for t in tensors:
        if t.device.type != "cuda" or t.device != t0.device:
            raise ValueError("all rank buffers must be on the same GPU")
        if t.dtype != t0.dtype or t.numel() != t0.numel():
            raise ValueError("rank buffers must share dtype and length")
        if not t.is_contiguous():
            raise ValueError("rank buffers must be contiguous")
    ptrs = (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    return ptrs, t0.numel(), _TORCH_DTYPES[t0.dtype]


def allreduce_ring(tensors, op: str = "sum", nslices: int = 1, *, stream=None, **opts) -> None:
    """In-place ring AllReduce over the list of R rank buffers (one per virtual rank)."""
    ptrs, count, dt = _buffers(tensors)
    with torch.cuda.device(tensors[0].device):
        s = _stream_handle(stream)
        if opts:
            o = _options(**opts)
            st = _allreduce_ring_ex(ptrs, len(tensors), count, DTYPES[dt], OPS[op], nslices,
                                    ctypes.byref(o), s)
        else:
            st = _allreduce_ring(ptrs, len(tensors), count, DTYPES[dt], OPS[op], nslices, s)
    _check(st, "allreduce_ring")


def allreduce_ring_timed(tensors, op: str = "sum", nslices: int = 1, *, stream=None, **opts):
    """allreduce_ring with a clock stamp per (lane, rank, hop).  Returns (stamps,
    clock_khz): stamps is a device tensor of shape (lanes, R, 2(R-1), 3) holding
    the wall clock when the wait for the hop began, when the hop's data movement
    began and when its arrival was sent (lanes = nslices * team of the plan)."""
    ptrs, count, dt = _buffers(tensors)
    R = len(tensors)
    p = plan(R, count, dt, nslices, **opts)
    lanes = nslices * p["team"]
    stamps = torch.zeros((lanes, R, max(1, 2 * (R - 1)), 3), dtype=torch.int64,
                         device=tensors[0].device)
    khz = ctypes.c_uint32(0)
    with torch.cuda.device(tensors[0].device):
        o = _options(**opts)
        st = _allreduce_ring_timed(ptrs, R, count, DTYPES[dt], OPS[op], nslices, ctypes.byref(o),
                                   stamps.data_ptr(), stamps.numel(), ctypes.byref(khz),
                                   _stream_handle(stream))
    _check(st, "allreduce_ring_timed")
    return stamps, khz.value


def reduce_scatter_ring(tensors, op: str = "sum", nslices: int = 1, *, stream=None, **opts) -> None:
    """In-place ring ReduceScatter: afterwards rank r owns chunk (r + 1) mod R."""
    ptrs, count, dt = _buffers(tensors)
    with torch.cuda.device(tensors[0].device):
        s = _stream_handle(stream)
        if opts:
            o = _options(**opts)
            st = _reduce_scatter_ring_ex(ptrs, len(tensors), count, DTYPES[dt], OPS[op], nslices,
                                         ctypes.byref(o), s)
        else:
            st = _reduce_scatter_ring(ptrs, len(tensors), count, DTYPES[dt], OPS[op], nslices, s)
    _check(st, "reduce_scatter_ring")


def all_gather_ring(tensors, nslices: int = 1, *, stream=None, **opts) -> None:
    """In-place ring AllGather of chunk (r + 1) mod R of every rank r."""
    ptrs, count, dt = _buffers(tensors)
    with torch.cuda.device(tensors[0].device):
        s = _stream_handle(stream)
        if opts:
            o = _options(**opts)
            st = _all_gather_ring_ex(ptrs, len(tensors), count, DTYPES[dt], nslices,
                                     ctypes.byref(o), s)
        else:
            st = _all_gather_ring(ptrs, len(tensors), count, DTYPES[dt], nslices, s)
    _check(st, "all_gather_ring")


def _pair(send, recv, send_elems, recv_elems):
    """Pointer arrays for send/receive tensor lists (same device, dtype, sizes)."""
    if not send or len(send) != len(recv):
        raise ValueError("need one send and one receive buffer per rank")
    t0 = send[0]
    if t0.dtype not in _TORCH_DTYPES:
        raise TypeError(f"unsupported dtype {t0.dtype}")
    for t, n in [(t, send_elems) for t in send] + [(t, recv_elems) for t in recv]:
        if t.device.type != "cuda" or t.device != t0.device or t.dtype != t0.dtype:
            raise ValueError("all buffers must be on the same GPU with the same dtype")
        if t.numel() != n or not t.is_contiguous():
            raise ValueError("buffer has the wrong length or is not contiguous")
    sp = (ctypes.c_void_p * len(send))(*[t.data_ptr() for t in send])
    rp = (ctypes.c_void_p * len(recv))(*[t.data_ptr() for t in recv])
    return sp, rp, _TORCH_DTYPES[t0.dtype]


def allreduce_ring_staged(send, recv=None, op: str = "sum", nslices: int = 1, *, stream=None,
                          **opts):
    """Out-of-place AllReduce by the staged primitives (recv defaults to new
    tensors; pass recv=send for in place).  Returns recv."""
    if recv is None:
        recv = [torch.empty_like(t) for t in send]
    n = send[0].numel()
    sp, rp, dt = _pair(send, recv, n, n)
    with torch.cuda.device(send[0].device):
        o = _options(**opts)
        st = _allreduce_ring_staged(sp, rp, len(send), n, DTYPES[dt], OPS[op], nslices,
                                    ctypes.byref(o), _stream_handle(stream))
    _check(st, "allreduce_ring_staged")
    return recv


def allreduce_ring_staged_noalloc(send, recv, op: str = "sum", nslices: int = 1, *, stream=None,
                                  **opts):
    """allreduce_ring_staged without any device allocation by the library (its
    receive slots and signals live in a static device array; the caller passes
    the output tensors).  Returns recv."""
    n = send[0].numel()
    sp, rp, dt = _pair(send, recv, n, n)
    with torch.cuda.device(send[0].device):
        o = _options(**opts)
        st = _allreduce_ring_staged_noalloc(sp, rp, len(send), n, DTYPES[dt], OPS[op], nslices,
                                            ctypes.byref(o), _stream_handle(stream))
    _check(st, "allreduce_ring_staged_noalloc")
    return recv


def reduce_scatter(send, recv=None, op: str = "sum", nslices: int = 1, *, stream=None, **opts):
    """Standalone ReduceScatter: send[r] holds R blocks; recv[r] gets block r
    reduced over all ranks.  Returns recv."""
    R = len(send)
    total = send[0].numel()
    if total % R:
        raise ValueError("send buffers must hold R equal blocks")
    n = total // R
    if recv is None:
        recv = [torch.empty(n, dtype=send[0].dtype, device=send[0].device) for _ in range(R)]
    sp, rp, dt = _pair(send, recv, total, n)
    with torch.cuda.device(send[0].device):
        o = _options(**opts)
        st = _reduce_scatter(sp, rp, R, n, DTYPES[dt], OPS[op], nslices, ctypes.byref(o),
                             _stream_handle(stream))
    _check(st, "reduce_scatter")
    return recv


def all_gather(send, recv=None, nslices: int = 1, *, stream=None, **opts):
    """Standalone AllGather: recv[r] gets all R send blocks in rank order.
    Returns recv."""
    R = len(send)
    n = send[0].numel()
    if recv is None:
        recv = [torch.empty(R * n, dtype=send[0].dtype, device=send[0].device) for _ in range(R)]
    sp, rp, dt = _pair(send, recv, n, R * n)
    with torch.cuda.device(send[0].device):
        o = _options(**opts)
        st = _all_gather(sp, rp, R, n, DTYPES[dt], nslices, ctypes.byref(o),
                         _stream_handle(stream))
    _check(st, "all_gather")
    return recv


def alltoall(send, recv=None, *, stream=None, **opts):
    """AlltoAll: send[r] and recv[r] hold R blocks; recv[q] block r = send[r]
    block q.  Returns recv."""
    R = len(send)
    total = send[0].numel()
    if total % R:
        raise ValueError("buffers must hold R equal blocks")
    if recv is None:
        recv = [torch.empty_like(t) for t in send]
    sp, rp, dt = _pair(send, recv, total, total)
    with torch.cuda.device(send[0].device):
        o = _options(**opts)
        st = _alltoall(sp, rp, R, total // R, DTYPES[dt], ctypes.byref(o), _stream_handle(stream))
    _check(st, "alltoall")
    return recv


def staged_ptrs(kind: str, send, recv, n: int, dtype, op="sum", nslices: int = 1, stream=0,
                **opts) -> int:
    """Raw-pointer call of the staged entry points; returns the status."""
    R = len(send) if send is not None else 0
    sp = (ctypes.c_void_p * max(1, R))(*send) if send is not None else None
    rp = (ctypes.c_void_p * max(1, len(recv)))(*recv) if recv is not None else None
    o = _options(**opts)
    dt = DTYPES.get(dtype, dtype if isinstance(dtype, int) else 99)
    opc = OPS.get(op, op if isinstance(op, int) else 99)
    if kind == "allreduce":
        return _allreduce_ring_staged(sp, rp, R, n, dt, opc, nslices, ctypes.byref(o), stream)
    if kind == "allreduce_noalloc":
        return _allreduce_ring_staged_noalloc(sp, rp, R, n, dt, opc, nslices, ctypes.byref(o),
                                              stream)
    if kind == "reduce_scatter":
        return _reduce_scatter(sp, rp, R, n, dt, opc, nslices, ctypes.byref(o), stream)
    if kind == "alltoall":
        return _alltoall(sp, rp, R, n, dt, ctypes.byref(o), stream)
    return _all_gather(sp, rp, R, n, dt, nslices, ctypes.byref(o), stream)


def allreduce_ring_ptrs(ptrs, count: int, dtype: str, op: str = "sum", nslices: int = 1,
                        stream=0, phase: str = "allreduce", **opts) -> int:
    """Raw-pointer call; returns the status instead of raising (argument tests)."""
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs) if ptrs is not None else None
    o = _options(**opts)
    R = len(ptrs) if ptrs is not None else 0
    if phase == "allreduce":
        return _allreduce_ring_ex(arr, R, count, DTYPES.get(dtype, dtype if isinstance(dtype, int) else 99),
                                  OPS.get(op, op if isinstance(op, int) else 99), nslices,
                                  ctypes.byref(o), stream)
    if phase == "reduce_scatter":
        return _reduce_scatter_ring_ex(arr, R, count, DTYPES[dtype], OPS[op], nslices,
                                       ctypes.byref(o), stream)
    return _all_gather_ring_ex(arr, R, count, DTYPES[dtype], nslices, ctypes.byref(o), stream)


def plan(R: int, count: int, dtype: str, nslices: int = 1, phase: str = "allreduce", **opts) -> dict:
    """The launch plan a call with these arguments would run (needs a GPU)."""
    p = _Plan()
    o = _options(**opts)
    _check(_plan_query(R, count, DTYPES[dtype], nslices, PHASES[phase], ctypes.byref(o),
                       ctypes.byref(p)), "rr_plan_query")
    d = {f: getattr(p, f) for f, _ in p._fields_}
    d["sync"] = SYNC_NAMES[d["sync"]]
    return d


def last_kernel_error(stream=None):
    """(status, record dict or None) of the device's failure record; clears it."""
    rec = ErrorRecord()
    st = _last_kernel_error(_stream_handle(stream), ctypes.byref(rec))
    return st, (rec.as_dict() if st == RR_ERR_TIMEOUT else None)


def check_kernel_error(stream=None) -> None:
    """Raise RRError if any device wait failed since the last check."""
    st, rec = last_kernel_error(stream)
    if st != RR_OK:
        raise RRError(st, "device wait", rec)


def init() -> None:
    _check(_init(), "rr_init")


def finalize() -> None:
    _finalize()


def workspace_preset(value: int, stream=None) -> None:
    _check(_workspace_preset(value, _stream_handle(stream)), "rr_workspace_preset")


def hbm_copy(dst, src, stream=None) -> None:
    """dst <- src with the library's streaming copy kernel (byte copy of src)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("destination too small")
    _check(_hbm_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream_handle(stream)), "rr_hbm_copy")


class CountingBarrier:
    """A set of counting signals: ``ncontexts`` x ``nwaiters``, 64-bit each."""

    def __init__(self, nwaiters: int, ncontexts: int = 1):
        h = ctypes.c_void_p()
        _check(_cb_create(nwaiters, ncontexts, ctypes.byref(h)), "counting_barrier_create")
        self._h = h
        self.nwaiters = nwaiters
        self.ncontexts = ncontexts

    @staticmethod
    def _mode(R, mode, expected, opts):
        """mode: barrier (a signal per waiter), shared (one per context), per_peer, p2p."""
        if mode == "shared":
            opts = dict(opts)
            opts["flags"] = opts.get("flags", 0) | FLAG_SHARED_SIGNAL
            mode = "barrier"
            if expected is None:
                expected = R
        if expected is None:
            expected = R - 1 if mode == "barrier" else 1  # p2p and per_peer: 1 per slot
        return mode, expected, opts

    def run(self, R: int, nsteps: int, ncontexts: int = 1, expected: int | None = None,
            mode: str = "barrier", stream=None, **opts) -> None:
        mode, expected, opts = self._mode(R, mode, expected, opts)
        o = _options(sync=mode, **opts)
        _check(_cb_run(self._h, R, nsteps, ncontexts, expected, ctypes.byref(o),
                       _stream_handle(stream)), "counting_barrier_run")

    def run_timed(self, R: int, nsteps: int, ncontexts: int = 1, expected: int | None = None,
                  mode: str = "barrier", stream=None, **opts):
        """``run`` with in-kernel timestamps.  Returns (stamps, clock_khz): stamps
        is a uint64 tensor on the GPU of shape (ncontexts, R, nsteps + 1), the
        device's constant-rate clock before each waiter's first step and when each
        of its steps' waits was over (valid once the stream has synchronised)."""
        mode, expected, opts = self._mode(R, mode, expected, opts)
        dev = torch.device("cuda", torch.cuda.current_device())
        stamps = torch.zeros((ncontexts, R, nsteps + 1), dtype=torch.int64, device=dev)
        khz = ctypes.c_uint32()
        o = _options(sync=mode, **opts)
        _check(_cb_run_timed(self._h, R, nsteps, ncontexts, expected, ctypes.byref(o),
                             stamps.data_ptr(), ctypes.byref(khz), _stream_handle(stream)),
               "counting_barrier_run_timed")
        return stamps, khz.value

    def read(self, ctx: int, waiter: int):
        v, s = _u64(), _u64()
        _check(_cb_read(self._h, ctx, waiter, ctypes.byref(v), ctypes.byref(s)),
               "counting_barrier_read")
        return v.value, s.value

    def read_peer(self, ctx: int, waiter: int, peer: int):
        """(slot value, shadow) of ``peer``'s per-peer slot in ``waiter``'s row."""
        v, s = _u64(), _u64()
        _check(_cb_read_peer(self._h, ctx, waiter, peer, ctypes.byref(v), ctypes.byref(s)),
               "counting_barrier_read_peer")
        return v.value, s.value

    def early_passes(self, ctx: int, waiter: int) -> int:
        n = _u64()
        _check(_cb_early(self._h, ctx, waiter, ctypes.byref(n)), "counting_barrier_early_passes")
        return n.value

    def reset(self, stream=None) -> None:
        _check(_cb_reset(self._h, _stream_handle(stream)), "counting_barrier_reset")

    def preset(self, value: int, stream=None) -> None:
        _check(_cb_preset(self._h, value, _stream_handle(stream)), "counting_barrier_preset")

    def close(self) -> None:
        if self._h:
            _check(_cb_destroy(self._h), "counting_barrier_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


@dataclass
class Slabs:
    """R rank buffers carved from one allocation, each 16-byte aligned, with
    guard words between them (so a stray write past a buffer is detectable)."""
    storage: torch.Tensor
    ranks: list
    stride: int


def make_slabs(R: int, count: int, dtype: torch.dtype, device="cuda", guard_bytes: int = 256,
               fill=None) -> Slabs:
    esize = torch.tensor([], dtype=dtype).element_size()
    per = (count * esize + guard_bytes + 255) // 256 * 256 // esize  # elements per slab stride
    storage = torch.empty(R * per + guard_bytes // esize, dtype=dtype, device=device)
    if fill is not None:
        storage.fill_(fill)
    ranks = [storage[r * per: r * per + count] for r in range(R)]
    return Slabs(storage, ranks, per)
