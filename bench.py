"""Benchmark: ring AllReduce over R virtual ranks on one MI355X.

Default workload: R=16 virtual ranks, fp32, 1 GiB per rank, SUM, 16 slices,
counting-barrier step sync (every rank adds 1 to each other rank's signal of the
lane after each hop; each waiter expects R-1).  One step is one in-place
AllReduce call (2(R-1) ring hops) over all R rank buffers, inputs resident in
HBM.  The rank buffers are separate tensors, as a caller's are (--layout slab
carves them from one allocation instead, 256 bytes apart).

Timing: W untimed calls, then exactly K timed calls.  Before every call the
inputs are restored from a pristine device copy, outside that call's pair of
HIP events on the launch stream, so every timed call reduces the workload's own
data.  ms_per_step is the median of the K per-call times.

value = algorithmic HBM bytes per call / time per call, with the algorithmic
bytes of the in-place ring: each ReduceScatter hop reads the incoming and local
chunk and writes the folded one (3 chunk transfers), each AllGather hop reads and
writes one chunk (2), so B = 5 (R-1) N for N bytes per rank.

Prints one JSON line.  Also reports:
  roofline         -- the ring kernel against MI355X's 8 TB/s HBM peak: its
                      average launch duration (the mean per-call event time over
                      the timed calls); `traffic` from the rocprofv3
                      FETCH_SIZE/WRITE_SIZE record in profiles/ when it was taken
                      on this kernel source, with the rate those counter bytes
                      give; the fraction of the same run's copy ceiling;
  extra_workloads  -- the other benchmark workloads (R=8 fp32 64 MiB, R=8 bf16
                      256 MiB, R=64 fp32 32 MiB), timed the same way;
  cpu_baseline     -- the single-threaded CPU oracle on the same inputs (test
                      infrastructure; timed only, never on the product path),
                      whose result is compared with the last timed GPU call,
                      every element of every rank;
  copy_ceiling     -- the library's streaming copy kernel over 1 GiB + 1 GiB.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of MI355X peak) for ring AllReduce over R virtual ranks"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD public specification
# timed after the headline in the same run (ring path), each with its own plan
EXTRA_WORKLOADS = ("r8_fp32_64MiB", "r8_bf16_256MiB", "r64_fp32_32MiB")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="r16_fp32_1GiB",
                    help="r16_fp32_1GiB | r8_fp32_64MiB | r8_bf16_256MiB | r64_fp32_32MiB | "
                         "worked_example | r16_sweep:K[:op[:nslices]]")
    ap.add_argument("--sync", default=None, help="auto | p2p | barrier | launch")
    ap.add_argument("--team", type=int, default=0)
    ap.add_argument("--block", type=int, default=0)
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--depth", type=int, default=0,
                    help="lanes each workgroup interleaves (0: the automatic plan)")
    ap.add_argument("--rounds", type=int, default=0,
                    help="lane groups each workgroup runs one after another (0: automatic)")
    ap.add_argument("--path", default="ring",
                    choices=["ring", "staged", "reduce_scatter", "all_gather", "alltoall"],
                    help="ring: the in-place ring (headline); staged: the out-of-place staged "
                         "primitives; reduce_scatter / all_gather: the standalone collectives "
                         "over the same per-rank buffer (R blocks / one block per rank); "
                         "alltoall: the per-rank buffer as R blocks, one per receiver")
    ap.add_argument("--fused", action="store_true",
                    help="fuse the last ReduceScatter hop with the first AllGather hop")
    ap.add_argument("--layout", default="separate", choices=("separate", "slab"),
                    help="rank buffers as separate tensors (default) or carved from one "
                         "allocation 256 bytes apart")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other benchmark workloads (ring path only)")
    ap.add_argument("--r16-sweep", action="store_true",
                    help="R=16 fp32 size sweep, 4 KiB .. 1 GiB per rank: one JSON line per point")
    ap.add_argument("--host-cost", action="store_true",
                    help="instead of the AllReduce: host time to enqueue one call (through "
                         "the C ABI) beside the GPU time of the call, at 8, 16 and 64 ranks "
                         "and small to mid sizes, with and without the per-call pointer checks")
    ap.add_argument("--hop-timeline", action="store_true",
                    help="instead of the headline: one call of the workload with a clock stamp "
                         "per (lane, rank, hop) (allreduce_ring_timed), summarised as wait "
                         "and move times per hop and the spread of hop ends across ranks")
    ap.add_argument("--order-ab", action="store_true",
                    help="instead of the headline: the in-place ring with the automatic hop "
                         "order against every hop ascending, interleaved in one process, "
                         "over R = 2..64 and 1 MiB..1 GiB per rank (one JSON line per point)")
    ap.add_argument("--barrier-latency", action="store_true",
                    help="instead of the AllReduce: per-step latency of the counting barrier "
                         "alone for R = 2..64 and 1 or 8 contexts (one JSON line per point)")
    return ap.parse_args()


def rank_buffers(rr, torch, R, count, dtype, layout):
    """The R rank buffers and a snapshot function (call it once, after filling the
    buffers; it returns a function that copies the inputs back).

    separate: one tensor per rank, as a caller's buffers normally are (torch's
              caching allocator puts large tensors 2 MiB apart);
    slab:     R buffers carved from one allocation 256 bytes apart (the layout
              the parity tests use, with guard bands to catch stray stores)."""
    if layout == "slab":
        slabs = rr.make_slabs(R, count, dtype, device="cuda")
        ranks = slabs.ranks

        def snapshot():
            saved = slabs.storage.clone()
            return lambda: slabs.storage.copy_(saved)
    else:
        ranks = [torch.empty(count, dtype=dtype, device="cuda") for _ in range(R)]

        def snapshot():
            saved = [t.clone() for t in ranks]

            def restore():
                for t, v in zip(ranks, saved):
                    t.copy_(v)
            return restore
    return ranks, snapshot


def pick_workload(name):
    import workloads
    if name.startswith("r16_sweep:"):
        parts = name.split(":")
        k = int(parts[1])
        op = parts[2] if len(parts) > 2 else "sum"
        ns = int(parts[3]) if len(parts) > 3 else 4
        return workloads.r16_sweep(k, op, ns)
    return workloads.ALL[name]


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ring_allreduce_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload_name, digest):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE for this
    kernel source (profiles/traffic_<workload>.json), or None if stale/absent."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != digest:
        return None
    return rec.get("traffic_bytes_per_launch")


def _torch_types(torch, np, dtype):
    tdt = {"int32": torch.int32, "fp32": torch.float32, "bf16": torch.bfloat16,
           "fp16": torch.float16}[dtype]
    two = dtype in ("bf16", "fp16")
    return tdt, (torch.int16 if two else torch.int32), (np.int16 if two else np.int32)


class Run:
    """One workload on one path: the rank buffers filled from the seeded inputs,
    a pristine copy of them, and the call that makes one step."""

    def __init__(self, rr, torch, np, w, path, opts, layout):
        import workloads
        self.rr, self.torch, self.w, self.path = rr, torch, w, path
        self.blk = w.count // w.R
        t = time.time()
        self.x = workloads.inputs(w)
        log(f"{w.name}: inputs generated in {time.time() - t:.1f} s")
        tdt, raw_t, raw_np = _torch_types(torch, np, w.dtype)
        self.raw_t, self.raw_np = raw_t, raw_np
        ranks, snapshot = rank_buffers(rr, torch, w.R, w.count, tdt, layout)
        for r in range(w.R):
            ranks[r].view(raw_t).copy_(torch.from_numpy(self.x[r].view(raw_np)))
        self.ranks = ranks
        # in place (the ring): every call must start from the inputs again
        self.restore = snapshot() if path == "ring" else (lambda: None)
        blk = self.blk
        if path == "ring":
            self.out = ranks
            self.call = lambda: rr.allreduce_ring(ranks, w.op, w.nslices, **opts)
        elif path == "staged":
            self.out = [torch.empty(w.count, dtype=tdt, device="cuda") for _ in range(w.R)]
            self.call = lambda: rr.allreduce_ring_staged(ranks, self.out, w.op, w.nslices, **opts)
        elif path == "reduce_scatter":
            self.out = [torch.empty(blk, dtype=tdt, device="cuda") for _ in range(w.R)]
            self.call = lambda: rr.reduce_scatter(ranks, self.out, w.op, w.nslices, **opts)
        elif path == "all_gather":
            send = [t[:blk] for t in ranks]
            self.out = [torch.empty(w.count, dtype=tdt, device="cuda") for _ in range(w.R)]
            self.call = lambda: rr.all_gather(send, self.out, w.nslices, **opts)
        else:
            self.out = [torch.empty(w.count, dtype=tdt, device="cuda") for _ in range(w.R)]
            self.call = lambda: rr.alltoall(ranks, self.out)

    def time(self, steps, warmup):
        """W untimed calls, then exactly K timed calls.  Before every call the
        inputs are restored from the pristine copy, outside that call's pair of
        HIP events (recorded on the launch stream); the output left behind is
        that of the last timed call, made from the inputs like every other."""
        torch, rr = self.torch, self.rr
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            self.restore()
            self.call()
        torch.cuda.synchronize()
        rr.check_kernel_error()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in evs:
            self.restore()
            e0.record(stream)
            self.call()
            e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        rr.check_kernel_error()
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        srt = sorted(ms)
        return {"calls": len(ms), "median_ms": round(srt[len(srt) // 2], 5),
                "mean_ms": round(sum(ms) / len(ms), 5), "min_ms": round(srt[0], 5),
                "max_ms": round(srt[-1], 5), "wall_s": round(wall, 3)}, ms

    def release(self):
        self.ranks = self.out = self.x = self.call = self.restore = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def _phase(path):
    return {"ring": "allreduce", "staged": "allreduce_staged",
            "reduce_scatter": "reduce_scatter_blocks", "all_gather": "all_gather_blocks",
            "alltoall": "alltoall"}[path]


def _plan_for(rr, w, path, opts):
    n = w.count // w.R if path in ("reduce_scatter", "all_gather", "alltoall") else w.count
    return rr.plan(w.R, n, w.dtype, w.nslices, phase=_phase(path),
                   **({} if path == "alltoall" else opts))


def _opts_for(w, path, args):
    opts = dict(sync=w.sync, team=args.team, block=args.block, flags=args.flags,
                fused=args.fused, depth=args.depth, rounds=args.rounds)
    if path != "ring":
        opts.pop("depth")
        if w.sync == "barrier":
            opts["sync"] = "auto"  # the staged loop is paced by its credits
        opts.pop("fused")
    return opts


def copy_ceiling(rr, torch):
    """The library's streaming copy over 1 GiB -> 1 GiB, and torch's elementwise
    add over 1 GiB fp32 operands (2 reads + 1 write, the shape of a
    ReduceScatter hop) as a reference."""
    stream = torch.cuda.current_stream()
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        rr.hbm_copy(dst, src)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    reps = 10
    for _ in range(reps):
        rr.hbm_copy(dst, src)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    out = {"bytes": 2 * n, "ms": round(ms, 4), "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}
    fa = src.view(torch.float32)
    fb = dst.view(torch.float32)
    fc = torch.empty_like(fa)
    for _ in range(3):
        torch.add(fa, fb, out=fc)
    a.record(stream)
    for _ in range(reps):
        torch.add(fa, fb, out=fc)
    b.record(stream)
    torch.cuda.synchronize()
    ms2 = a.elapsed_time(b) / reps
    out["read2_write1"] = {"bytes": 3 * n, "ms": round(ms2, 4),
                           "GB/s": round(3 * n / (ms2 * 1e-3) / 1e9, 1),
                           "kernel": "torch.add (reference)"}
    del src, dst, fc
    torch.cuda.empty_cache()
    return out


def cpu_baseline(run, np, budget_s):
    """The oracle (test infrastructure, this leg only) on the same inputs: timed
    on one host core over whole calls until the budget is spent (at least one
    call), each call on a fresh copy of the inputs (the copy is not timed).  Its
    result is then compared with the GPU output of the last timed call, every
    element of every rank, one piece of each rank buffer at a time."""
    import oracle
    w, path, x = run.w, run.path, run.x
    blk = run.blk
    runs, spent, expect = 0, 0.0, None
    work = None
    while runs == 0 or spent < budget_s:
        if path == "ring":
            if work is None:
                work = [np.empty_like(a) for a in x]
            for a, b in zip(work, x):
                np.copyto(a, b)
            t = time.perf_counter()
            oracle.allreduce(work, w.op)
            spent += time.perf_counter() - t
            expect = work
        else:
            t = time.perf_counter()
            if path == "staged":
                expect, _ = oracle.staged_allreduce(x, w.op)
            elif path == "reduce_scatter":
                expect, _ = oracle.reduce_scatter_nccl(x, w.op)
            elif path == "alltoall":
                expect = oracle.alltoall(x)
            else:
                expect, _ = oracle.all_gather_nccl([np.ascontiguousarray(a[:blk]) for a in x])
            spent += time.perf_counter() - t
        runs += 1
    per = spent / runs
    # every element of every rank, a piece at a time (bounded host memory)
    piece = 1 << 26
    ok = True
    for r in range(w.R):
        dev = run.out[r].view(run.raw_t)
        want = expect[r].view(run.raw_np)
        for lo in range(0, want.size, piece):
            hi = min(lo + piece, want.size)
            got = dev[lo:hi].cpu().numpy()
            if not np.array_equal(got, want[lo:hi]):
                ok = False
                break
        if not ok:
            break
    return per, runs, spent, ok


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the virtual ranks of the ring all live in one "
              "MI355X's HBM, and the library has no path across GPUs. Use --gpus 1.",
              file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    import ring_allreduce_amd as rr

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.barrier_latency:
        return barrier_latency(rr, torch, np)
    if args.host_cost:
        return host_cost(rr, torch)
    if args.r16_sweep:
        return r16_sweep(rr, torch, np, args.layout)
    if args.order_ab:
        return order_ab(rr, torch)
    w = pick_workload(args.workload)
    if args.sync:
        w = w.with_(sync=args.sync)
    if args.hop_timeline:
        return hop_timeline(rr, torch, np, w, args)
    path = args.path
    opts = _opts_for(w, path, args)
    if path != "ring" and w.count % w.R:
        print("the standalone collectives need a per-rank count divisible by R", file=sys.stderr)
        return 2
    rr.init()
    p = _plan_for(rr, w, path, opts)
    log(f"workload {w.name} ({path}): R={w.R} {w.dtype} {w.op} "
        f"{w.bytes_per_rank / 2**20:.1f} MiB/rank nslices={w.nslices} plan={p}")
    kernel = {"ring": "ring_kernel", "alltoall": "alltoall_kernel"}.get(path, "staged_kernel")

    run = Run(rr, torch, np, w, path, opts, args.layout)
    timing, per_call = run.time(args.steps, args.warmup)
    B = p["hbm_bytes"]
    ms_per_step = timing["median_ms"]
    value = B / (ms_per_step * 1e-3) / 1e9
    log(f"timed {args.steps} calls: median {ms_per_step:.4f} ms, mean {timing['mean_ms']:.4f} ms "
        f"-> {value:.1f} GB/s algorithmic")

    # The kernel's average launch duration: the mean of the per-call HIP event
    # times on the launch stream, divided by the launches one call makes.
    per_call_launches = p["launches"]
    avg_launch_ms = timing["mean_ms"] / per_call_launches
    bytes_per_launch = B / per_call_launches
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    digest = source_digest()
    traffic = stored_traffic(w.name if path == "ring" else f"{path}_{w.name}", digest)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kernel, "launch_ms_avg": round(avg_launch_ms, 5),
                "launches_timed": args.steps * per_call_launches,
                "bytes_per_launch": int(bytes_per_launch), "kernel_source_digest": digest}
    if traffic:
        # what the counters saw leave the L2s (Infinity Cache hits included)
        cgbs = traffic / (avg_launch_ms * 1e-3) / 1e9
        roofline["counter_GBps"] = round(cgbs, 1)
        roofline["counter_frac"] = round(cgbs / HBM_PEAK_GBS, 4)

    extra = {}
    if path == "ring" and not args.no_extra:
        for name in EXTRA_WORKLOADS:
            if name == w.name:
                continue
            wx = workloads_all()[name]
            ox = dict(sync=wx.sync)  # each with its own automatic plan
            px = _plan_for(rr, wx, "ring", ox)
            rx = Run(rr, torch, np, wx, "ring", ox, args.layout)
            tx, _ = rx.time(args.steps, args.warmup)
            rx.release()
            bx = px["hbm_bytes"]
            gbs = bx / (tx["median_ms"] * 1e-3) / 1e9
            extra[name] = {"ms": tx["median_ms"], "mean_ms": tx["mean_ms"],
                           "min_ms": tx["min_ms"], "max_ms": tx["max_ms"],
                           "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                           "sync": px["sync"], "block": px["block"], "depth": px["depth"],
                           "rounds": px["rounds"], "team": px["team"],
                           "algorithmic_bytes": bx}
            log(f"extra {name}: {extra[name]}")

    ceiling = None
    if not args.no_copy_ceiling:
        ceiling = copy_ceiling(rr, torch)
        roofline["frac_of_copy_ceiling"] = round(achieved / ceiling["GB/s"], 4)
        log(f"copy ceiling: {ceiling}")

    cpu = None
    if not args.no_cpu_baseline:
        per, runs, spent, ok = cpu_baseline(run, np, args.cpu_seconds)
        cpu = {"value": round(B / per / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "ms_per_call": round(per * 1e3, 1),
               "sample": f"the full {w.name} input, {runs} call(s) of the single-threaded C "
                         f"oracle ({spent:.1f} s), each on a fresh copy of the inputs",
               "gpu_matches_oracle_bitwise": bool(ok),
               "compared": "every element of every rank: the output of the last timed call",
               "host_cpu": _cpu_model(), "host_nproc": os.cpu_count()}
        cpu["gpu_over_cpu"] = round(value / cpu["value"], 1)
        log(f"cpu baseline: {cpu}")
    run.release()

    out = {
        "metric": METRIC if path == "ring" else f"{METRIC} ({path} path)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic", "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "config": {"workload": w.name, "path": path, "R": w.R, "bytes_per_rank": w.bytes_per_rank,
                   "op": w.op, "nslices": w.nslices, "sync": p["sync"], "team": p["team"],
                   "block": p["block"], "grid": p["grid"], "launches_per_step": p["launches"],
                   "rounds": p["rounds"], "depth": p["depth"], "stream_loads": p["stream_loads"],
                   "alternate": p["alternate"],
                   "fused_boundary": bool(p["fused"]) if path == "ring" else False,
                   "algorithmic_bytes_per_step": B, "layout": args.layout,
                   "inputs_restored_before_each_call": path == "ring",
                   "parallelism": "virtual ranks on 1 GPU"},
        "timing": timing,
        # the ring's traffic in the sources' sense: bytes sent over all links per call
        "bus_bytes_per_step": (2 * (w.R - 1) * w.bytes_per_rank if path in ("ring", "staged")
                               else (w.R - 1) * w.bytes_per_rank),
        "roofline": roofline, "cpu_baseline": cpu, "copy_ceiling": ceiling,
        "extra_workloads": extra or None,
    }
    print(json.dumps(out), flush=True)
    return 0


def workloads_all():
    import workloads
    return workloads.ALL


def hop_timeline(rr, torch, np, w, args):
    """Where a call's time goes, hop by hop.  After the warm-up calls (inputs
    restored before each), one call of the workload through allreduce_ring_timed:
    every (lane, rank, hop) gets the device clock when its workgroup began to wait
    for the hop's hand-off, when the wait was over and when the hop's arrival was
    sent.  Printed (one JSON line): the call's span; per hop, the median time
    moving data and waiting; the share of workgroup time spent waiting; how far
    apart the ranks of a lane end the same hop (median and 90th percentile over
    lanes and hops)."""
    opts = _opts_for(w, "ring", args)
    opts.pop("fused")
    rr.init()
    run = Run(rr, torch, np, w, "ring", opts, args.layout)
    run.time(max(1, args.steps // 4), args.warmup)
    run.restore()
    stamps, khz = rr.allreduce_ring_timed(run.ranks, w.op, w.nslices, **opts)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    st = stamps.cpu().numpy().astype(np.float64) * (1e3 / khz)  # microseconds
    run.release()
    t0, t1, t2 = st[..., 0], st[..., 1], st[..., 2]             # (lanes, R, hops)
    start = t0[:, :, 0].min()
    wait = (t1 - t0)[:, :, 1:]
    move = t2 - t1
    spread = t2.max(axis=1) - t2.min(axis=1)                    # (lanes, hops)
    busy = (t2 - t0)[:, :, 1:].sum()
    pct = lambda a, q: round(float(np.percentile(a, q)), 2)
    p = rr.plan(w.R, w.count, w.dtype, w.nslices, **opts)
    print(json.dumps({
        "metric": "hop timeline", "workload": w.name, "sync": p["sync"],
        "flags": args.flags, "block": p["block"], "team": p["team"], "depth": p["depth"],
        "rounds": p["rounds"], "lanes": int(st.shape[0]), "hops": int(st.shape[2]),
        "span_us": round(float(t2.max() - start), 1),
        "move_us_per_lane_hop": {"p10": pct(move, 10), "p50": pct(move, 50),
                                 "p90": pct(move, 90)},
        "wait_us_per_lane_hop": {"p50": pct(wait, 50), "p90": pct(wait, 90),
                                 "p99": pct(wait, 99)},
        "wait_share_of_busy_time": round(float(wait.sum() / busy), 4),
        "hop_end_spread_across_ranks_us": {"p50": pct(spread, 50), "p90": pct(spread, 90)},
        "clock_khz": khz}), flush=True)
    return 0


def host_cost(rr, torch):
    """Host microseconds per call: the time the C ABI takes to validate, plan and
    enqueue one in-place AllReduce (ctypes call included, measured over 200
    calls issued back to back in batches of 20 with a synchronisation between
    batches, outside the timed part), beside the GPU time of one call (HIP
    events, median of 20).  Each point is taken with the per-call pointer checks
    (the default) and without them (RR_FLAG_NO_POINTER_CHECK); rank buffers are
    separate tensors.  A call is enqueue-bound when the host time exceeds the
    GPU time."""
    import ctypes
    rr.init()
    stream = torch.cuda.current_stream()
    for R in (8, 16, 64):
        for kib in (4, 64, 1024, 16384):
            count = kib * 1024 // 4
            ranks = [torch.zeros(count, device="cuda") for _ in range(R)]
            ptrs = [t.data_ptr() for t in ranks]
            p = rr.plan(R, count, "fp32", 4, sync="p2p")
            row = {"metric": "host cost per call", "R": R, "bytes_per_rank": count * 4,
                   "nslices": 4, "sync": p["sync"], "grid": p["grid"]}
            for label, flags in (("checked", 0), ("unchecked", rr.FLAG_NO_POINTER_CHECK)):
                def call():
                    st = rr.allreduce_ring_ptrs(ptrs, count, "fp32", "max", 4,
                                                stream=stream.cuda_stream,
                                                sync="p2p", flags=flags)
                    if st != rr.RR_OK:
                        raise RuntimeError(rr.status_string(st))
                for _ in range(10):
                    call()
                torch.cuda.synchronize()
                spent, n = 0.0, 0
                for _ in range(10):
                    t0 = time.perf_counter()
                    for _ in range(20):
                        call()
                    spent += time.perf_counter() - t0
                    n += 20
                    torch.cuda.synchronize()
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(20)]
                for a, e in evs:
                    a.record(stream)
                    call()
                    e.record(stream)
                torch.cuda.synchronize()
                rr.check_kernel_error()
                gpu = sorted(a.elapsed_time(e) for a, e in evs)[10] * 1e3
                row[f"host_us_{label}"] = round(spent / n * 1e6, 2)
                row[f"gpu_us_{label}"] = round(gpu, 2)
            print(json.dumps(row), flush=True)
            del ranks
            torch.cuda.empty_cache()
    return 0


def barrier_latency(rr, torch, np):
    """Per-step latency of the barrier on its own, in three layouts: one 64-lane
    workgroup per (context, waiter); per step each waiter arrives and waits.
      barrier   counting signal: adds 1 to each other waiter's one signal, waits
                for its own to advance by R-1
      shared    one signal per context: every waiter adds 1 to it and waits for
                it to advance by R (the ring's default barrier layout)
      per_peer  per-peer slots: adds 1 to its own slot in each other waiter's
                row, waits for each of the R-1 slots of its row to advance by 1
      p2p       adds 1 to its successor's signal, waits for 1
    us/step = (t(nsteps) - t(0)) / nsteps, best of 5 timed launches each; beside it
    the in-kernel distribution of step times (the device clock stamped when each
    waiter's wait for each step is over) and the spread between the first and
    the last waiter of a context leaving the same step.  Then,
    for the counting barrier, audited runs count the steps a waiter passed on a
    stand-in arrival from a peer one step ahead (a lower bound)."""
    rr.init()
    b = rr.CountingBarrier(64, 8)
    stream = torch.cuda.current_stream()

    def timed(R, nsteps, nctx, mode):
        best = None
        for _ in range(5):
            a = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.run(R, nsteps, nctx, mode=mode)
            e.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(e)
            best = ms if best is None else min(best, ms)
        rr.check_kernel_error()
        return best

    steps = 2000
    for mode in ("barrier", "shared", "per_peer", "p2p"):
        for nctx in (1, 8):
            for R in (2, 4, 8, 16, 32, 64):
                b.run(R, 100, nctx, mode=mode)  # warm
                t0 = timed(R, 0, nctx, mode)
                t1 = timed(R, steps, nctx, mode)
                us = (t1 - t0) * 1e3 / steps
                per_waiter = 1 if mode in ("p2p", "shared") else R - 1
                # in-kernel view: each waiter's step times from the device clock, and
                # how far apart the waiters of a context leave the same step
                st, khz = b.run_timed(R, steps, nctx, mode=mode)
                torch.cuda.synchronize()
                rr.check_kernel_error()
                stamps = st.cpu().numpy()
                to_us = 1e3 / khz
                step_us = np.diff(stamps[:, :, 1:], axis=2).ravel() * to_us
                spread_us = (stamps[:, :, 1:].max(axis=1) - stamps[:, :, 1:].min(axis=1)).ravel() * to_us
                pct = lambda a, q: round(float(np.percentile(a, q)), 3)
                print(json.dumps({"metric": "barrier latency per step", "mode": mode,
                                  "R": R, "contexts": nctx, "us_per_step": round(us, 3),
                                  "atomics_per_step": nctx * R * per_waiter,
                                  "slots_per_waiter": 1 if mode != "per_peer" else R - 1,
                                  "empty_launch_ms": round(t0, 4),
                                  "in_kernel_step_us": {"p50": pct(step_us, 50),
                                                        "p90": pct(step_us, 90),
                                                        "p99": pct(step_us, 99),
                                                        "max": round(float(step_us.max()), 3)},
                                  "exit_spread_us": {"p50": pct(spread_us, 50),
                                                     "max": round(float(spread_us.max()), 3)},
                                  "clock_khz": khz}), flush=True)
    for R in (4, 8, 16, 64):
        nctx, asteps = 8, 500
        b.reset()
        b.run(R, asteps, nctx, mode="barrier", flags=rr.FLAG_AUDIT)
        torch.cuda.synchronize()
        rr.check_kernel_error()
        early = sum(b.early_passes(c, q) for c in range(nctx) for q in range(R))
        print(json.dumps({"metric": "counting barrier early passes (audited)", "R": R,
                          "contexts": nctx, "steps": asteps, "waits": nctx * R * asteps,
                          "early_passes": early}), flush=True)
    b.close()
    return 0


def r16_sweep(rr, torch, np, layout="separate"):
    """The R=16 fp32 sweep, 4 KiB * 4^k per rank (k = 0..9): SUM with 1, 2, 4, 8 and
    16 slices and MAX with 4, each in barrier and p2p mode.  Per point: 2 warm-up
    calls, then 10 calls, each after the inputs are restored (outside its events)
    and timed with its own HIP events on the launch stream; the median is
    reported.  GB/s on the algorithmic bytes 5(R-1)N."""
    import workloads
    rr.init()
    stream = torch.cuda.current_stream()
    for k in range(10):
        w0 = workloads.r16_sweep(k, "sum", 4)
        x = workloads.inputs(w0)
        ranks, restore = rank_buffers(rr, torch, w0.R, w0.count, torch.float32, layout)
        for r in range(w0.R):
            ranks[r].copy_(torch.from_numpy(x[r]))
        del x
        restore = restore()
        for op, ns in (("sum", 1), ("sum", 2), ("sum", 4), ("sum", 8), ("sum", 16), ("max", 4)):
            for sync in ("barrier", "p2p"):
                p = rr.plan(w0.R, w0.count, "fp32", ns, sync=sync)
                for _ in range(2):
                    restore()
                    rr.allreduce_ring(ranks, op, ns, sync=sync)
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(10)]
                for a, e in evs:
                    restore()
                    a.record(stream)
                    rr.allreduce_ring(ranks, op, ns, sync=sync)
                    e.record(stream)
                torch.cuda.synchronize()
                rr.check_kernel_error()
                times = sorted(a.elapsed_time(e) for a, e in evs)
                ms = times[len(times) // 2]
                B = p["hbm_bytes"]
                print(json.dumps({"metric": "R=16 fp32 sweep", "bytes_per_rank": w0.bytes_per_rank,
                                  "op": op, "nslices": ns, "sync": p["sync"], "ms": round(ms, 5),
                                  "min_ms": round(times[0], 5),
                                  "GB/s": round(B / ms / 1e6, 1),
                                  "pct_of_peak": round(100 * B / ms / 1e6 / HBM_PEAK_GBS, 2),
                                  "team": p["team"], "depth": p["depth"], "rounds": p["rounds"],
                                  "block": p["block"], "grid": p["grid"], "layout": layout,
                                  "stream_loads": p["stream_loads"], "alternate": p["alternate"],
                                  "launches": p["launches"]}),
                      flush=True)
        del ranks, restore
        torch.cuda.empty_cache()
    return 0


def order_ab(rr, torch):
    """The automatic hop order (even hops top down once the R buffers exceed
    128 MiB) against every hop ascending (RR_FLAG_ASCENDING), in one process on
    one set of buffers: fp32 SUM over R = 2..64 and 1 MiB..1 GiB per rank (up to
    16 GiB in all), bf16 at three points, both hand-off modes.  Per point and
    order: three repetitions, interleaved, of 2 warm-up and 5 timed calls, each
    after the inputs are restored outside its events; the median of the three
    medians is reported.  Uniform inputs in [-1, 1) from torch's generator."""
    rr.init()
    stream = torch.cuda.current_stream()
    cases = []
    for R in (2, 4, 8, 16, 32, 64):
        for mib in (1, 16, 64, 256, 1024):
            if R * mib > 16384 or (R >= 32 and mib > 256):
                continue
            for sync in ("p2p", "barrier"):
                cases.append((R, mib, "fp32", sync))
    for R, mib in ((8, 256), (16, 256), (64, 32)):
        for sync in ("p2p", "barrier"):
            cases.append((R, mib, "bf16", sync))
    for R, mib, dt, sync in cases:
        tdt = torch.float32 if dt == "fp32" else torch.bfloat16
        count = mib * (1 << 20) // (4 if dt == "fp32" else 2)
        ns = 16 if R == 16 else 8
        g = torch.Generator(device="cuda")
        g.manual_seed(R * 131 + mib)
        ranks, snapshot = rank_buffers(rr, torch, R, count, tdt, "separate")
        for t in ranks:
            t.uniform_(-1, 1, generator=g)
        restore = snapshot()
        p = rr.plan(R, count, dt, ns, sync=sync)
        orders = {"auto": dict(sync=sync), "ascending": dict(sync=sync, order="ascending")}
        med = {k: [] for k in orders}
        for _ in range(3):
            for k, o in orders.items():
                for _ in range(2):
                    restore()
                    rr.allreduce_ring(ranks, "sum", ns, **o)
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(5)]
                for a, e in evs:
                    restore()
                    a.record(stream)
                    rr.allreduce_ring(ranks, "sum", ns, **o)
                    e.record(stream)
                torch.cuda.synchronize()
                rr.check_kernel_error()
                med[k].append(sorted(a.elapsed_time(e) for a, e in evs)[2])
        ms = {k: sorted(v)[1] for k, v in med.items()}
        B = p["hbm_bytes"]
        print(json.dumps({"metric": "hop order A/B", "R": R, "bytes_per_rank": mib << 20,
                          "dtype": dt, "sync": p["sync"], "alternate": p["alternate"],
                          "team": p["team"], "depth": p["depth"], "rounds": p["rounds"],
                          "block": p["block"], "auto_ms": round(ms["auto"], 5),
                          "ascending_ms": round(ms["ascending"], 5),
                          "auto_pct": round(100 * B / ms["auto"] / 1e6 / HBM_PEAK_GBS, 2),
                          "ascending_pct": round(100 * B / ms["ascending"] / 1e6 / HBM_PEAK_GBS, 2),
                          "speedup": round(ms["ascending"] / ms["auto"], 4)}), flush=True)
        del ranks, restore
        torch.cuda.empty_cache()
    return 0


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    sys.exit(main())
