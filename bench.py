"""Benchmark: ring AllReduce over R virtual ranks on one MI355X.

Default workload: R=8 virtual ranks, fp32, 64 MiB per rank, SUM, 4 slices.  One
step is one in-place AllReduce call (2(R-1) ring hops) over all R rank buffers,
inputs resident in HBM.  The rank buffers are separate tensors, as a caller's
are (--layout slab carves them from one allocation instead, 256 bytes apart:
R=64 in barrier mode runs about 4% slower there).

value = algorithmic HBM bytes per call / time per call, with the algorithmic
bytes of the in-place ring: each ReduceScatter hop reads the incoming and local
chunk and writes the folded one (3 chunk transfers), each AllGather hop reads and
writes one chunk (2), so B = 5 (R-1) N for N bytes per rank.

Prints one JSON line (rank 0).  Also reports:
  roofline      -- the ring kernel against MI355X's 8 TB/s HBM peak: its average
                   launch duration from HIP events on the launch stream around the
                   timed region; `traffic` from the rocprofv3 FETCH_SIZE/WRITE_SIZE
                   record in profiles/ when it was taken on this kernel source;
  cpu_baseline  -- the single-threaded CPU oracle on the same inputs (test
                   infrastructure; timed only, never on the product path), which
                   also cross-checks one GPU call;
  copy_ceiling  -- the library's streaming copy kernel over 1 GiB + 1 GiB.
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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="r8_fp32_64MiB",
                    help="r8_fp32_64MiB | r8_bf16_256MiB | r64_fp32_32MiB | worked_example | "
                         "r16_sweep:K[:op[:nslices]]")
    ap.add_argument("--sync", default=None, help="auto | p2p | barrier | launch")
    ap.add_argument("--team", type=int, default=0)
    ap.add_argument("--block", type=int, default=0)
    ap.add_argument("--flags", type=int, default=0)
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
    ap.add_argument("--r16-sweep", action="store_true",
                    help="R=16 fp32 size sweep, 4 KiB .. 1 GiB per rank: one JSON line per point")
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
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.barrier_latency:
        return barrier_latency(rr, torch, np)
    if args.r16_sweep:
        return r16_sweep(rr, torch, np, args.layout)
    w = pick_workload(args.workload)
    if args.sync:
        w = w.with_(sync=args.sync)
    opts = dict(sync=w.sync, team=args.team, block=args.block, flags=args.flags,
                fused=args.fused)
    path = args.path
    if path != "ring":
        if w.sync == "barrier":
            opts["sync"] = "auto"  # the staged loop is paced by its credits
        opts.pop("fused")
        if w.count % w.R:
            print("the standalone collectives need a per-rank count divisible by R",
                  file=sys.stderr)
            return 2
    blk = w.count // w.R
    rr.init()
    phase = {"ring": "allreduce", "staged": "allreduce_staged",
             "reduce_scatter": "reduce_scatter_blocks", "all_gather": "all_gather_blocks",
             "alltoall": "alltoall"}[path]
    p = rr.plan(w.R, blk if path in ("reduce_scatter", "all_gather", "alltoall") else w.count,
                w.dtype, w.nslices, phase=phase,
                **({} if path == "alltoall" else opts))
    log(f"workload {w.name} ({path}): R={w.R} {w.dtype} {w.op} "
        f"{w.bytes_per_rank / 2**20:.1f} MiB/rank nslices={w.nslices} plan={p}")

    t = time.time()
    x = workloads.inputs(w)
    log(f"inputs generated in {time.time() - t:.1f} s")
    torch_dt = {"int32": torch.int32, "fp32": torch.float32, "bf16": torch.bfloat16,
                "fp16": torch.float16}[w.dtype]
    raw_t = torch.int16 if workloads.ELEM_BYTES[w.dtype] == 2 else torch.int32
    raw_np = np.int16 if workloads.ELEM_BYTES[w.dtype] == 2 else np.int32
    ranks, restore = rank_buffers(rr, torch, w.R, w.count, torch_dt, args.layout)
    for r in range(w.R):
        ranks[r].view(raw_t).copy_(torch.from_numpy(x[r].view(raw_np)))
    restore = restore()  # snapshot the inputs; calling it copies them back
    stream = torch.cuda.current_stream()
    kernel = {"ring": "ring_kernel", "alltoall": "alltoall_kernel"}.get(path, "staged_kernel")

    if path == "ring":
        out_bufs = ranks

        def step():
            rr.allreduce_ring(ranks, w.op, w.nslices, **opts)
    elif path == "staged":
        out_bufs = [torch.empty(w.count, dtype=torch_dt, device="cuda") for _ in range(w.R)]

        def step():
            rr.allreduce_ring_staged(ranks, out_bufs, w.op, w.nslices, **opts)
    elif path == "reduce_scatter":
        out_bufs = [torch.empty(blk, dtype=torch_dt, device="cuda") for _ in range(w.R)]

        def step():
            rr.reduce_scatter(ranks, out_bufs, w.op, w.nslices, **opts)
    elif path == "all_gather":
        ag_send = [t[:blk] for t in ranks]
        out_bufs = [torch.empty(w.count, dtype=torch_dt, device="cuda") for _ in range(w.R)]

        def step():
            rr.all_gather(ag_send, out_bufs, w.nslices, **opts)
    else:
        out_bufs = [torch.empty(w.count, dtype=torch_dt, device="cuda") for _ in range(w.R)]

        def step():
            rr.alltoall(ranks, out_bufs)

    # one checked call on the pristine inputs, kept for the CPU cross-check
    step()
    torch.cuda.synchronize()
    rr.check_kernel_error()
    first_result = [t.view(raw_t).cpu().numpy() for t in out_bufs]

    for _ in range(args.warmup):
        step()
    restore()
    torch.cuda.synchronize()
    rr.check_kernel_error()

    # timed region: exactly K steps
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    rr.check_kernel_error()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    B = p["hbm_bytes"]
    value = B / (ms_per_step * 1e-3) / 1e9
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step (wall {wall_ms / args.steps:.4f}) "
        f"-> {value:.1f} GB/s algorithmic")

    # Per-call spread: each of K further calls between its own pair of events
    # (outside the timed region above, so `value` is unaffected).
    per_call_ms = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    rr.check_kernel_error()
    per_call_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    timing = {"calls": len(per_call_ms), "median_ms": round(per_call_ms[len(per_call_ms) // 2], 5),
              "min_ms": round(per_call_ms[0], 5), "max_ms": round(per_call_ms[-1], 5)}

    # The ring kernel's average launch duration: HIP events on the launch stream
    # around the timed region, divided by the launches it holds (back to back).
    per_call = p["launches"]
    avg_launch_ms = ev0.elapsed_time(ev1) / (args.steps * per_call)
    bytes_per_launch = B / per_call
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    digest = source_digest()
    traffic = stored_traffic(w.name if path == "ring" else f"{path}_{w.name}", digest)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kernel, "launch_ms_avg": round(avg_launch_ms, 5),
                "launches_timed": args.steps * per_call, "bytes_per_launch": int(bytes_per_launch),
                "kernel_source_digest": digest}

    copy_ceiling = None
    if not args.no_copy_ceiling:
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
        copy_ceiling = {"bytes": 2 * n, "ms": round(ms, 4),
                        "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}
        # a 2-read + 1-write stream (the shape of a ReduceScatter hop): torch's
        # elementwise add over 1 GiB fp32 operands, as a reference only
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
        copy_ceiling["read2_write1"] = {"bytes": 3 * n, "ms": round(ms2, 4),
                                        "GB/s": round(3 * n / (ms2 * 1e-3) / 1e9, 1),
                                        "kernel": "torch.add (reference)"}
        del src, dst, fc
        log(f"copy ceiling: {copy_ceiling}")

    cpu_baseline = None
    if not args.no_cpu_baseline:
        import oracle  # test infrastructure: the CPU baseline leg only
        runs, spent = 0, 0.0
        expect = None
        while runs == 0 or (spent < args.cpu_seconds and runs < 1000):
            t = time.perf_counter()
            if path == "ring":
                bufs = [a.copy() for a in x]
                t = time.perf_counter()
                oracle.allreduce(bufs, w.op)
            elif path == "staged":
                bufs, _ = oracle.staged_allreduce(x, w.op)
            elif path == "reduce_scatter":
                bufs, _ = oracle.reduce_scatter_nccl(x, w.op)
            elif path == "alltoall":
                bufs = oracle.alltoall(x)
            else:
                bufs, _ = oracle.all_gather_nccl([np.ascontiguousarray(a[:blk]) for a in x])
            spent += time.perf_counter() - t
            runs += 1
            expect = bufs
        per = spent / runs
        ok = all(np.array_equal(first_result[r].view(np.uint8), expect[r].view(np.uint8))
                 for r in range(w.R))
        cpu_baseline = {"value": round(B / per / 1e9, 3), "unit": "GB/s", "cores": 1,
                        "kind": "oracle", "ms_per_call": round(per * 1e3, 1),
                        "sample": f"the full {w.name} input, {runs} call(s) of the single-threaded "
                                  f"C oracle ({spent:.1f} s)",
                        "gpu_matches_oracle_bitwise": bool(ok),
                        "host_cpu": _cpu_model(), "host_nproc": os.cpu_count()}
        log(f"cpu baseline: {cpu_baseline}")

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
                   "fused_boundary": bool(p["fused"]) if path == "ring" else False,
                   "algorithmic_bytes_per_step": B, "layout": args.layout,
                   "parallelism": "virtual ranks on 1 GPU"},
        "timing": timing,
        # ring traffic in the sources' sense: bytes sent over all links per call
        "bus_bytes_per_step": (2 * (w.R - 1) * w.bytes_per_rank if path in ("ring", "staged")
                               else (w.R - 1) * w.bytes_per_rank),
        "roofline": roofline, "cpu_baseline": cpu_baseline, "copy_ceiling": copy_ceiling,
    }
    print(json.dumps(out), flush=True)
    return 0


def barrier_latency(rr, torch, np):
    """Per-step latency of the barrier on its own, in three layouts: one 64-lane
    workgroup per (context, waiter); per step each waiter arrives and waits.
      barrier   counting signal: adds 1 to each other waiter's one signal, waits
                for its own to advance by R-1
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
    for mode in ("barrier", "per_peer", "p2p"):
        for nctx in (1, 8):
            for R in (2, 4, 8, 16, 32, 64):
                b.run(R, 100, nctx, mode=mode)  # warm
                t0 = timed(R, 0, nctx, mode)
                t1 = timed(R, steps, nctx, mode)
                us = (t1 - t0) * 1e3 / steps
                per_waiter = 1 if mode == "p2p" else R - 1
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
    16 slices and MAX with 4, each in barrier and p2p mode.  Per point: inputs
    restored, 2 warm-up calls, then 10 calls timed with HIP events on the launch
    stream; GB/s on the algorithmic bytes 5(R-1)N."""
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
                restore()
                for _ in range(2):
                    rr.allreduce_ring(ranks, op, ns, sync=sync)
                a = torch.cuda.Event(enable_timing=True)
                e = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(10):
                    rr.allreduce_ring(ranks, op, ns, sync=sync)
                e.record(stream)
                torch.cuda.synchronize()
                rr.check_kernel_error()
                ms = a.elapsed_time(e) / 10
                B = p["hbm_bytes"]
                print(json.dumps({"metric": "R=16 fp32 sweep", "bytes_per_rank": w0.bytes_per_rank,
                                  "op": op, "nslices": ns, "sync": p["sync"], "ms": round(ms, 5),
                                  "GB/s": round(B / ms / 1e6, 1),
                                  "pct_of_peak": round(100 * B / ms / 1e6 / HBM_PEAK_GBS, 2),
                                  "team": p["team"], "depth": p["depth"], "rounds": p["rounds"],
                                  "block": p["block"], "grid": p["grid"], "layout": layout,
                                  "stream_loads": p["stream_loads"], "launches": p["launches"]}),
                      flush=True)
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
