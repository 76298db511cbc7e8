#!/usr/bin/env python3
"""Benchmark of the barrier-free AllReduce on one MI355X with emulated ranks.

    python bench.py [--steps K] [--warmup W] [--workload 2] [--all --report out.json]

Default workload: 4 emulated ranks, bf16 sum, one-shot sentinel with double buffering, messages
of 1 KiB .. 256 KiB per rank (powers of two). A step is one AllReduce of every message size of
the workload; K steps run back to back inside one persistent launch per size (no host work
between iterations), each iteration on a fresh input set. Per iteration k the latency is
max_r t_end[r][k] - max_r t_start[r][k] on the device wall clock (from the moment the last rank
enters until the last rank has completed its last output store). The JSON line reports the p50,
the on-chip latency floor 2 * L_L2 + L_store measured in the same run, the roofline of the
dominant kernel (algorithmic bytes per launch / launch time from HIP events on the launch
stream) and the single-threaded CPU oracle on a bounded sample.

Only one GPU is used: ranks are emulated on it. ``--gpus`` above 1 is refused.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "p50 AllReduce latency µs @128B–1MB; algBW GB/s @≥16MB (1 GPU)"
HBM_PEAK_GBPS = 8000.0


def _to_device(x):
    import torch

    out = []
    for r in range(x.shape[0]):
        row = np.ascontiguousarray(x[r])
        if row.dtype == np.uint16:
            row = row.view(np.int16)
        out.append(torch.from_numpy(row).cuda())
    return out


def bench_size(A, I, h, wid: int, wl: dict, size_idx: int, size: int, algo: str, iters: int,
               warmup: int, hz: float, set_cap_bytes: int = 256 << 20, check: bool = True):
    import torch

    n, dt = wl["nranks"], wl["dtype"]
    eb = I.ELEM_BYTES[dt]
    count = size // eb
    # the standalone collectives: `size` is the per-rank partition; inputs and outputs differ
    in_count = n * count if algo == "reducescatter" else count
    out_count = n * count if algo == "allgather" else count
    io_bytes = max(in_count, out_count) * eb
    nsets = max(1, min(iters, set_cap_bytes // (n * io_bytes)))
    host_sets = []
    if n * io_bytes <= (8 << 20):
        xs = []
        for k in range(nsets):
            x = I.rank_inputs(wl["dist"], dt, n, in_count, wid, size_idx, k, wl["sigma"])
            I.assert_finite(x, dt)
            xs.append(x)
        if check:
            host_sets.append((nsets - 1, xs[-1]))
        # one contiguous [nsets, count] buffer per rank: set k of rank r is a slice, so the
        # sets are evenly spaced and the persistent loop addresses them without a table
        big = [torch.from_numpy(np.ascontiguousarray(
            np.stack([xs[k][r] for k in range(nsets)]).view(
                np.int16 if dt == "bf16" else xs[0].dtype))).cuda() for r in range(n)]
        del xs
    else:
        big = [t.view(1, -1) for t in
               I.device_draw(wl["dist"], dt, n, in_count, wid, size_idx, 0, wl["sigma"])]
        nsets = 1
    outs_big = [torch.empty((nsets, out_count), dtype=b.dtype, device=b.device) for b in big]
    ins = [big[r][k] for k in range(nsets) for r in range(n)]
    outs = [outs_big[r][k] for k in range(nsets) for r in range(n)]
    torch.cuda.synchronize()
    aid = A.ALGOS[algo]
    # Untimed pass over every input set first: the timed iterations then find the sets where the
    # preceding computation would have left them (in the caches while they fit).
    warm = max(warmup, nsets)
    if warm > 0:
        A.ar_bench(h, ins, outs, nsets, count, aid, warm, timestamps=False)
    ts, te, ms = A.ar_bench_ex(h, ins, outs, nsets, count, aid, iters)
    # launch-inclusive: host-issued ar_allreduce calls back to back, timed with events
    calls = 50
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def one_call():
        if algo == "reducescatter":
            A.ar_reducescatter(h, ins[:n], outs[:n], count)
        elif algo == "allgather":
            A.ar_allgather(h, ins[:n], outs[:n], count)
        elif algo == "broadcast":
            A.ar_broadcast(h, ins[0], outs[:n], count, 0)
        else:
            A.ar_allreduce(h, ins[:n], outs[:n], count, aid)

    one_call()
    ev0.record()
    for _ in range(calls):
        one_call()
    ev1.record()
    torch.cuda.synchronize()
    launch_us = ev0.elapsed_time(ev1) * 1e3 / calls
    ts = ts.reshape(iters, n).astype(np.int64)
    te = te.reshape(iters, n).astype(np.int64)
    lat_us = (te.max(axis=1) - ts.max(axis=1)) / hz * 1e6
    ends = te.max(axis=1)
    period_us = float((ends[-1] - ends[0]) / (iters - 1) / hz * 1e6) if iters > 1 else float("nan")
    res = {
        "bytes": size,
        "count": count,
        "p50_us": float(np.percentile(lat_us, 50)),
        "p99_us": float(np.percentile(lat_us, 99)),
        "mean_us": float(lat_us.mean()),
        "period_us": period_us,
        "launch_ms": float(ms),
        "launch_inclusive_us": float(launch_us),
        "iters": iters,
        "alg_bytes_per_call": A.ar_alg_bytes(h, count, aid),
        "launch": A.ar_plan_info(h, count, aid),
    }
    res["algbw_GBps"] = size / (res["p50_us"] * 1e-6) / 1e9
    res["busbw_like_GBps"] = res["alg_bytes_per_call"] * iters / (ms * 1e-3) / 1e9 if ms > 0 else 0
    if check and host_sets:
        # spot check: the last set's output equals the oracle's result (the parity tests proper
        # live in tests/)
        from oracle import oracle

        k, x = host_sets[-1]
        rows = [np.ascontiguousarray(x[r]) for r in range(n)]
        if algo in I.COLLECTIVES:
            want_all = (oracle.reducescatter(rows) if algo == "reducescatter"
                        else oracle.allgather(rows) if algo == "allgather"
                        else oracle.broadcast(rows[0], n))
            ok = all(np.array_equal(outs[k * n + r].cpu().numpy().view(np.uint8),
                                    want_all[r].view(np.uint8)) for r in range(n))
            res["spot_check"] = bool(ok)
            if not ok:
                raise AssertionError(f"spot check failed: {algo} n={n} size={size}")
            del ins, outs, big, outs_big
            return res
        want = oracle.allreduce(rows)[0]
        got = outs[k * n].cpu().numpy().view(want.dtype)
        if algo == "ll128_atomic":
            ok = np.allclose(got.astype(np.float64), want.astype(np.float64), rtol=0,
                             atol=float(n * 2.0 ** -23 * np.abs(x.astype(np.float64)).sum(0).max()))
        else:
            ok = np.array_equal(got.view(np.uint8), want.view(np.uint8))
        res["spot_check"] = bool(ok)
        if not ok:
            raise AssertionError(f"spot check failed: {algo} n={n} size={size}")
    del ins, outs, big, outs_big
    return res


def copy_peak(A, mib: int = 1024, reps: int = 5) -> dict:
    """Achievable HBM bandwidth on this machine: the library's streaming copy over `mib` MiB, every
    byte read once and written once, timed with events on the stream it runs on."""
    import torch

    nbytes = mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    A.ar_stream_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        A.ar_stream_copy(dst, src, nbytes)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    del src, dst
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms,
            "GBps": 2 * nbytes / (ms * 1e-3) / 1e9}


def kernel_source_hash() -> str:
    """sha256 over the HIP sources and the C header: counters taken on another version of the
    kernels do not describe this one."""
    import glob
    import hashlib

    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "latency_collectives_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "ar.h"))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload_key: str):
    """HBM bytes per timed launch from the committed counter summary (profiles/traffic.json),
    or None when there is none for this workload or the kernels have changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec


def cpu_baseline(I, wid: int, wl: dict, budget_s: float = 12.0) -> dict:
    """The oracle as it stands, single-threaded, timed on this host on the workload's sizes."""
    from oracle import oracle

    n, dt = wl["nranks"], wl["dtype"]
    sizes = wl["sizes"]
    per_size = []
    per_budget = budget_s / len(sizes)
    for si, size in enumerate(sizes):
        count = size // I.ELEM_BYTES[dt]
        x = I.rank_inputs(wl["dist"], dt, n, count, wid, si, 0, wl["sigma"])
        rows = [np.ascontiguousarray(x[r]) for r in range(n)]
        t1 = oracle.time_allreduce(rows, 1)
        reps = max(1, min(100000, int(per_budget / max(t1, 1e-7))))
        t = oracle.time_allreduce(rows, reps)
        per_size.append({"bytes": size, "reps": reps, "us_per_call": t / reps * 1e6})
    gm = math.exp(sum(math.log(p["us_per_call"]) for p in per_size) / len(per_size))
    return {
        "value": gm,
        "unit": "us",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"single-threaded C++ oracle (left fold, -O2), {n} ranks {dt}, each of the "
                   f"{len(sizes)} message sizes repeated for ~{per_budget:.1f} s; value = "
                   "geometric mean over sizes of the mean time per AllReduce"),
        "host_threads_available": os.cpu_count(),
        "per_size": per_size,
    }


def cpu_baseline_threads(I, wid: int, wl: dict, threads: int, budget_s: float = 6.0) -> dict:
    """The same oracle run on `threads` host threads at once, each on an equal slice of the
    element range of every rank (the C call releases the interpreter lock); the rank order per
    element is unchanged, so the result is the same. Reported beside the single-threaded value."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle

    n, dt = wl["nranks"], wl["dtype"]
    sizes = wl["sizes"]
    per_budget = budget_s / len(sizes)
    per_size = []
    with ThreadPoolExecutor(max_workers=threads) as pool:
        for si, size in enumerate(sizes):
            count = size // I.ELEM_BYTES[dt]
            x = I.rank_inputs(wl["dist"], dt, n, count, wid, si, 0, wl["sigma"])
            rows = [np.ascontiguousarray(x[r]) for r in range(n)]
            t = min(threads, count)
            cuts = [count * j // t for j in range(t + 1)]
            slices = [[row[cuts[j]:cuts[j + 1]] for row in rows] for j in range(t)]
            t0 = time.perf_counter()
            list(pool.map(lambda sl: oracle.time_allreduce(sl, 1), slices))
            one = max(time.perf_counter() - t0, 1e-7)
            reps = max(1, min(100000, int(per_budget / one)))
            t0 = time.perf_counter()
            list(pool.map(lambda sl: oracle.time_allreduce(sl, reps), slices))
            per_size.append({"bytes": size, "reps": reps, "threads": t,
                             "us_per_call": (time.perf_counter() - t0) / reps * 1e6})
    gm = math.exp(sum(math.log(p["us_per_call"]) for p in per_size) / len(per_size))
    return {"value": gm, "unit": "us", "cores": threads, "per_size": per_size}


def run_workload(A, I, wid: int, algo: str | None, iters: int | None, warmup: int, hz: float,
                 placement: int, sizes=None):
    wl = dict(I.WORKLOADS[wid])
    if sizes is not None:
        wl["sizes"] = sizes
    algo = algo or wl["algo"]
    iters = iters or wl["iters"]
    # reduce-scatter inputs and all-gather outputs are N partitions per rank
    widen = wl["nranks"] if algo in ("reducescatter", "allgather") else 1
    h = A.ar_create(wl["nranks"], max(wl["sizes"]) * widen, A.DTYPES[wl["dtype"]])
    try:
        A.ar_set_option(h, A.AR_OPT_PLACEMENT, placement)
        rows = []
        for si, size in enumerate(wl["sizes"]):
            rows.append(bench_size(A, I, h, wid, wl, si, size, algo, iters, warmup, hz))
            print(f"# workload {wid} {algo} size {size}: p50 {rows[-1]['p50_us']:.3f} us "
                  f"p99 {rows[-1]['p99_us']:.3f} us", file=sys.stderr, flush=True)
    finally:
        A.ar_destroy(h)
    return wl, algo, iters, rows


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed iterations per size")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=sorted([1, 2, 3, 4, 5, 6, 7, 8]))
    ap.add_argument("--algo", default=None)
    ap.add_argument("--placement", type=int, default=0, help="0 XCD per rank, 1 same XCD")
    ap.add_argument("--all", action="store_true", help="also run every workload; see --report")
    ap.add_argument("--auto-sweep", action="store_true",
                    help="only measure the one-shot / two-shot crossovers behind AR_ALGO_AUTO")
    ap.add_argument("--report", default=None, help="write the full per-size report here")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-barrier-baseline", action="store_true")
    ap.add_argument("--sizes", default=None,
                    help="comma-separated message sizes in bytes (default: the workload's)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run the streaming copy kernel over MIB MiB (5 times) and exit; "
                         "its known byte count scales rocprof FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the ranks are emulated on a single MI355X; "
              f"--gpus {args.gpus} (world size {world}) is not supported.", file=sys.stderr)
        return 2

    import torch

    from latency_collectives_amd import _ar as A
    from latency_collectives_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        A.ar_stream_copy(dst, src, nbytes)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(5):
            A.ar_stream_copy(dst, src, nbytes)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / 5
        print(json.dumps({"calibrate_copy_bytes_read": nbytes, "bytes_written": nbytes,
                          "ms_per_copy": ms, "GBps_read_plus_write": 2 * nbytes / ms / 1e6}),
              flush=True)
        return 0
    hz = A.ar_wallclock_hz()
    if args.auto_sweep:
        rows = auto_sweep(A, I, hz, args.warmup, args.placement)
        print(json.dumps({"auto_sweep": rows}), flush=True)
        return 0
    sol = A.ar_sol_ex(args.placement)
    print(f"# sol {json.dumps(sol)}", file=sys.stderr, flush=True)
    peak = copy_peak(A)
    print(f"# streaming copy {peak['GBps']:.0f} GB/s", file=sys.stderr, flush=True)

    wid = args.workload
    sizes = [int(x) for x in args.sizes.split(",")] if args.sizes else None
    wl, algo, iters, rows = run_workload(A, I, wid, args.algo, args.steps, args.warmup, hz,
                                         args.placement, sizes)
    p50s = [r["p50_us"] for r in rows]
    value = math.exp(sum(math.log(v) for v in p50s) / len(p50s))
    barrier = None
    if algo != "barrier2" and algo not in I.COLLECTIVES and not args.no_barrier_baseline:
        # the two-barrier baseline at the same sizes, same inputs, same run
        _, _, _, brows = run_workload(A, I, wid, "barrier2", args.steps, args.warmup, hz,
                                      args.placement, sizes)
        bp50 = [r["p50_us"] for r in brows]
        barrier = {
            "algo": "barrier2",
            "value": math.exp(sum(math.log(v) for v in bp50) / len(bp50)),
            "unit": "us",
            "p50_us": [round(v, 4) for v in bp50],
            "p99_us": [round(r["p99_us"], 4) for r in brows],
        }
    total_launch_ms = sum(r["launch_ms"] for r in rows)
    floor_us = sol["floor_ns"] * 1e-3
    # Dominant kernel: the one this workload runs; roofline over all its timed launches.
    tot_bytes = sum(r["alg_bytes_per_call"] * r["iters"] for r in rows)
    achieved = tot_bytes / (total_launch_ms * 1e-3) / 1e9
    launches = len(rows)
    tkey = f"workload{wid}:{algo}:{wl['dtype']}:" + ",".join(str(x) for x in wl["sizes"]) + \
        f":steps{iters}"
    traffic_rec = measured_traffic(tkey)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "us",
        "n_gpus": 1,
        "steps": iters,
        "warmup": args.warmup,
        "ms_per_step": total_launch_ms / iters,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic",
        "config": {
            "workload": (f"{wl['nranks']} emulated ranks on one MI355X, {wl['dtype']} sum "
                         f"(fp32 accumulation), {algo}, {min(wl['sizes'])}-{max(wl['sizes'])} "
                         f"bytes per rank (powers of two), {iters} back-to-back iterations per "
                         "size, fresh inputs per iteration"),
            "nranks": wl["nranks"],
            "algo": algo,
            "placement": ["rank per XCD", "all ranks on one XCD"][args.placement],
            "sizes_bytes": wl["sizes"],
        },
        "value_definition": ("geometric mean over the message sizes of the per-size p50 "
                             "latency (device wall clock, last rank in to last rank out)"),
        "per_size": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                     for r in rows],
        "latency_floor": {
            "floor_us": floor_us,
            "formula": "2*L_L2 + L_store (dependent-load L2 latency; store->poll half RTT)",
            "l2_load_ns": sol["l2_load_ns"],
            "store_half_rtt_ns": sol["store_half_rtt_ns"],
            "fence_ns": sol["fence_ns"],
            "p50_smallest_over_floor": p50s[0] / floor_us,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": (traffic_rec["hbm_bytes_per_launch"] if traffic_rec else None),
            "alg_bytes_per_launch": tot_bytes / launches,
            "launches": launches,
            "mean_launch_ms": total_launch_ms / launches,
            "kernel": f"ar_kernel<{algo}, {wl['dtype']}, N={wl['nranks']}>",
            "bytes_definition": ("ar_alg_bytes() per AllReduce x iterations per launch; achieved = "
                                 "bytes over all timed launches / their summed event time"),
            "traffic_definition": ("rocprofv3 FETCH_SIZE + WRITE_SIZE per timed launch, each "
                                   "scaled by the streaming copy's counter-to-bytes factor "
                                   "(profiles/traffic.json); null when the kernel sources "
                                   "differ from those the counters were taken on"),
            "copy_peak_GBps": peak["GBps"],
            "frac_of_copy_peak": achieved / peak["GBps"],
        },
    }
    if barrier is not None:
        line["barrier_baseline"] = barrier
    if not args.no_cpu_baseline and algo not in I.COLLECTIVES:
        line["cpu_baseline"] = cpu_baseline(I, wid, wl)
        # the machine's CPU share is 16 cores whatever os.cpu_count() reports
        line["cpu_baseline"]["multi_thread"] = cpu_baseline_threads(
            I, wid, wl, max(1, min(16, os.cpu_count() or 1)))
    report = {"main": line, "sol": sol}
    if args.all:
        report["workloads"] = run_all(A, I, hz, args.warmup, args.placement)
    if args.report:
        with open(args.report, "w") as f:
            json.dump(report, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


def auto_sweep(A, I, hz, warmup, placement, iters=100):
    """p50 of the one-shot LL, one-shot sentinel and two-shot kernels for N in {2,3,4,8,16} and
    per-rank sizes 128 B .. 2 MiB (fp32, uniform inputs): the measurements behind the automatic
    algorithm choice (ar_allreduce with AR_ALGO_AUTO)."""
    sizes = [128 << (2 * k) for k in range(7)] + [2 << 20]
    out = []
    for n in (2, 3, 4, 8, 16):
        wl = dict(nranks=n, dtype="f32", dist="uniform", sigma=1.0, sizes=sizes)
        h = A.ar_create(n, max(sizes), A.AR_FLOAT32)
        try:
            A.ar_set_option(h, A.AR_OPT_PLACEMENT, placement)
            for si, size in enumerate(sizes):
                row = {"nranks": n, "bytes": size}
                for algo in ("oneshot_ll", "oneshot_sentinel", "twoshot"):
                    r = bench_size(A, I, h, 6, wl, si, size, algo, iters, warmup, hz)
                    row[algo] = round(r["p50_us"], 3)
                best = min(("oneshot_ll", "oneshot_sentinel", "twoshot"), key=lambda a: row[a])
                row["best"] = best
                print(f"# sweep {json.dumps(row)}", file=sys.stderr, flush=True)
                out.append(row)
        finally:
            A.ar_destroy(h)
    return out


def run_all(A, I, hz, warmup, placement):
    out = {}
    plan = [
        (1, ["oneshot_ll", "oneshot_sentinel", "barrier2"]),
        (2, ["oneshot_sentinel", "oneshot_ll", "twoshot", "barrier2"]),
        (3, ["twoshot", "oneshot_sentinel", "barrier2"]),
        (4, ["ll128_atomic", "oneshot_ll", "oneshot_sentinel", "twoshot", "barrier2"]),
        (5, ["twoshot"]),
        (6, ["reducescatter"]),
        (7, ["allgather"]),
        (8, ["broadcast"]),
    ]
    for wid, algos in plan:
        for algo in algos:
            wl, algo, iters, rows = run_workload(A, I, wid, algo, None, warmup, hz, placement)
            out[f"{wid}:{algo}:{wl['dtype']}"] = rows
        if wid == 5:
            wl = dict(I.WORKLOADS[5], dtype="f32", dist="uniform")
            h = A.ar_create(8, max(wl["sizes"]), A.AR_FLOAT32)
            try:
                rows = [bench_size(A, I, h, 5, wl, si, s, "twoshot", wl["iters"], warmup, hz)
                        for si, s in enumerate(wl["sizes"])]
            finally:
                A.ar_destroy(h)
            out["5:twoshot:f32"] = rows
    # barrier latency versus N (one cross-rank barrier per iteration)
    bar = []
    for n in (2, 4, 8, 16):
        h = A.ar_create(n, 16, A.AR_FLOAT32)
        try:
            A.ar_set_option(h, A.AR_OPT_PLACEMENT, placement)
            A.ar_bench(h, None, None, 1, 0, A.AR_BARRIER_ONLY, 50)
            _, _, ms = A.ar_bench_ex(h, None, None, 1, 0, A.AR_BARRIER_ONLY, 2000)
            bar.append({"nranks": n, "us_per_barrier": ms * 1e3 / 2000})
        finally:
            A.ar_destroy(h)
    out["barrier_only"] = bar
    return out


if __name__ == "__main__":
    sys.exit(main())
