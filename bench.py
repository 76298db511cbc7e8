#!/usr/bin/env python3
"""Benchmark of the barrier-free AllReduce on one MI355X with emulated ranks.

    python bench.py [--steps K] [--warmup W] [--configs 1,2,3,4,5] [--report out.json]

A step is one AllReduce of every message size of every configuration below (all five are
measured in the default run); K steps run back to back inside one persistent launch per
(configuration, algorithm, size), each iteration on a fresh input set where the sets fit in
memory. Per iteration k the latency is max_r t_end[r][k] - max_r t_start[r][k] on the device
wall clock (from the moment the last rank enters until the last rank has completed its last
output store).

    1  oneshot_ll_n2_f32_128B: 2 ranks, fp32, 128 B, one-shot LL (also the one-shot sentinel and
       the two-barrier baseline)
    2  oneshot_sentinel_n4_bf16_1K-256K: 4 ranks, bf16, 1 KiB - 256 KiB, one-shot sentinel +
       double buffering                                                   <- `value`
    3  twoshot_n8_bf16_tp_decode_8192: 8 ranks, bf16, [tokens, 8192] for tokens 1..64
       (16 KiB - 1 MiB), two-shot (and the one-shot for comparison)
    4  ll128_vs_oneshot_vs_barrier_n16_f32_4K-4M: 16 ranks, fp32, 4 KiB - 4 MiB, LL128-style
       atomic vs one-shot LL vs two-barrier baseline
    5  twoshot_n8_bandwidth_16M-256M: 8 ranks, int32 and fp32, 16 - 256 MiB, two-shot (bandwidth
       regime: algBW = S / p50)

The JSON line's `value` is the geometric mean of the 4-rank bf16 workload's per-size p50;
`configs` holds every workload's per-size p50 / p99, its latency roofline (p50 against the
on-chip floor 2 * L_L2 + L_store of the slowest XCD pair the workload uses, plus its algorithmic
bytes at 8 TB/s) or, for the bandwidth workload, its HBM roofline; `roofline` is the headline
kernel's. The CPU oracle is timed on a bounded sample of the headline workload
(`cpu_baseline`).

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

# Workload id in inputs.WORKLOADS -> (algorithms measured, extra dtypes). The first algorithm is
# the one the workload names; the others run at the same sizes for comparison.
CONFIGS = {
    1: (["oneshot_ll", "oneshot_sentinel", "barrier2"], []),
    2: (["oneshot_sentinel", "barrier2"], []),
    3: (["twoshot", "oneshot_sentinel"], []),
    4: (["ll128_atomic", "oneshot_ll", "barrier2"], []),
    5: (["twoshot"], ["f32"]),
}
HEADLINE = 2  # `value`: the 4-rank bf16 one-shot sentinel workload
SPLIT = None  # --split: force the peer-split kernels on (1) or off (0); None = library default
BANDWIDTH = 5  # reported against the HBM roofline

# Kernel dispatches of the AllReduce kernels made so far by this process (ar_bench and every
# ar_allreduce / collective call is one dispatch): lets a rocprofv3 trace be matched to the
# per-size records (`dispatch` in each record is the index of its timed launch).
_DISPATCHES = [0]


def _gm(xs):
    xs = [x for x in xs if x and x > 0]
    return math.exp(sum(math.log(v) for v in xs) / len(xs)) if xs else float("nan")


def bench_size(A, I, h, wid: int, wl: dict, size_idx: int, size: int, algo: str, iters: int,
               warmup: int, hz: float, set_cap_bytes: int = 256 << 20, check: bool = True,
               launch_calls: int = 20, group: int = 4):
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
        _DISPATCHES[0] += 1
    dispatch = _DISPATCHES[0]
    ts, te, ms = A.ar_bench_ex(h, ins, outs, nsets, count, aid, iters)
    _DISPATCHES[0] += 1
    # launch-inclusive: host-issued calls back to back, timed with events
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
        _DISPATCHES[0] += 1

    launch_us = float("nan")
    if launch_calls > 0:
        one_call()
        ev0.record()
        for _ in range(launch_calls):
            one_call()
        ev1.record()
        torch.cuda.synchronize()
        launch_us = ev0.elapsed_time(ev1) * 1e3 / launch_calls
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
        "nsets": nsets,
        "dispatch": dispatch,
        "alg_bytes_per_call": A.ar_alg_bytes(h, count, aid),
        "launch": A.ar_plan_info(h, count, aid),
    }
    res["algbw_GBps"] = size / (res["p50_us"] * 1e-6) / 1e9
    res["alg_GBps_event"] = (res["alg_bytes_per_call"] * iters / (ms * 1e-3) / 1e9
                             if ms > 0 else 0.0)
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
        else:
            want = (oracle.allreduce_grouped(rows, group)[0]
                    if algo == "ll128_det" and dt != "i32" else oracle.allreduce(rows)[0])
            ok = True
            for r in range(n):
                got = outs[k * n + r].cpu().numpy().view(want.dtype)
                if algo == "ll128_atomic" and dt == "f32":
                    # per element: |gpu - oracle| <= N * 2^-23 * sum_r |x_r[i]|
                    bound = n * 2.0 ** -23 * np.abs(x.astype(np.float64)).sum(0)
                    ok &= bool(np.all(np.abs(got.astype(np.float64) - want.astype(np.float64))
                                      <= bound))
                elif algo == "ll128_atomic" and dt == "bf16":
                    # bf16 accumulation: N * 2^-8 * sum_r |x_r[i]| (plus N subnormal spacings)
                    def wide(b):
                        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                    bound = n * 2.0 ** -8 * np.abs(wide(x)).sum(0) + n * 2.0 ** -133
                    ok &= bool(np.all(np.abs(wide(got) - wide(want)) <= bound))
                else:
                    ok &= bool(np.array_equal(got.view(np.uint8), want.view(np.uint8)))
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
    """sha256 over the HIP sources (kernels, planner, launch code): counters taken on another
    version of them do not describe this one. The C header's text is documentation and is not
    part of it."""
    import glob
    import hashlib

    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "latency_collectives_amd", "csrc", "*")))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()


_TRAFFIC = {}


def traffic_table() -> dict:
    """Counter-measured HBM bytes per AllReduce, keyed by config:algo:dtype:n<N>:<bytes>
    (profiles/traffic.json), or {} when the kernels have changed since they were taken."""
    if "t" not in _TRAFFIC:
        path = os.path.join(ROOT, "profiles", "traffic.json")
        try:
            with open(path) as f:
                rec = json.load(f)
        except (OSError, ValueError):
            rec = {}
        ok = rec.get("source_sha256") == kernel_source_hash()
        _TRAFFIC["t"] = rec.get("entries", {}) if ok else {}
    return _TRAFFIC["t"]


def traffic_key(workload: str, algo: str, dtype: str, n: int, size: int) -> str:
    return f"{workload}:{algo}:{dtype}:n{n}:{size}"


def measured_traffic(cfg: str, algo: str, dtype: str, n: int, rows: list):
    """HBM bytes per timed launch (mean over the rows' launches) from the per-AllReduce counter
    record of every size, or None when any size has none."""
    t = traffic_table()
    per_launch = []
    for r in rows:
        e = t.get(traffic_key(cfg, algo, dtype, n, r["bytes"]))
        if e is None:
            return None
        per_launch.append(e["hbm_bytes_per_ar"] * r["iters"])
    return sum(per_launch) / len(per_launch)


# Dependent cross-rank exchanges on an algorithm's critical path: a one-shot pushes once; a
# two-shot (and the LL128-style kernel) reduce-scatters and then all-gathers, each phase waiting
# for the previous one's data; the barrier baseline is charged its data exchange only (the
# barriers are the cost it exists to show).
EXCHANGES = {"oneshot_ll": 1, "oneshot_sentinel": 1, "barrier2": 1, "twoshot": 2,
             "ll128_atomic": 2, "ll128_det": 2}


def latency_roofline(rows: list, floor_us: float, exchanges: int = 1) -> dict:
    """Latency roofline of a small-message configuration: per size the bound is `exchanges`
    times the on-chip floor plus the algorithmic bytes at the nominal HBM bandwidth (the floor
    term dominates below ~4 KiB); `frac` = bound / p50 (geometric mean over the sizes; 1 would
    be at the bound)."""
    bounds = [exchanges * floor_us + r["alg_bytes_per_call"] / (HBM_PEAK_GBPS * 1e9) * 1e6
              for r in rows]
    ratios = [r["p50_us"] / b for r, b in zip(rows, bounds)]
    return {
        "bound": "latency",
        "unit": "us",
        "achieved": _gm([r["p50_us"] for r in rows]),
        "peak": _gm(bounds),
        "frac": _gm([1.0 / x for x in ratios]),
        "p50_over_bound": [round(x, 3) for x in ratios],
        "bound_us": [round(b, 4) for b in bounds],
        "exchanges": exchanges,
        "bound_definition": ("exchanges * floor_us + alg_bytes_per_call / 8 TB/s per size; floor "
                             "= 2*L_L2 + L_store of the slowest sender->receiver XCD pair of the "
                             "placement; exchanges = dependent cross-rank exchanges of the "
                             "algorithm (1 one-shot, 2 two-shot)"),
    }


def hbm_roofline(rows: list, copy_gbps: float) -> dict:
    """HBM roofline of the dominant kernel: algorithmic bytes per launch / launch time (HIP
    events on the launch stream), against the nominal 8 TB/s and the streaming copy."""
    tot_bytes = sum(r["alg_bytes_per_call"] * r["iters"] for r in rows)
    tot_ms = sum(r["launch_ms"] for r in rows)
    achieved = tot_bytes / (tot_ms * 1e-3) / 1e9
    return {
        "bound": "hbm",
        "unit": "GB/s",
        "achieved": achieved,
        "peak": HBM_PEAK_GBPS,
        "frac": achieved / HBM_PEAK_GBPS,
        "alg_bytes_per_launch": tot_bytes / len(rows),
        "launches": len(rows),
        "mean_launch_ms": tot_ms / len(rows),
        "copy_peak_GBps": copy_gbps,
        "frac_of_copy_peak": achieved / copy_gbps,
        "per_size_GBps": [round(r["alg_GBps_event"], 1) for r in rows],
    }


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
    return {
        "value": _gm([p["us_per_call"] for p in per_size]),
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
    return {"value": _gm([p["us_per_call"] for p in per_size]), "unit": "us", "cores": threads,
            "per_size": per_size}


def run_workload(A, I, wid: int, algo: str | None, iters: int | None, warmup: int, hz: float,
                 placement: int, sizes=None, dtype: str | None = None, launch_calls: int = 20,
                 group: int | None = None):
    wl = dict(I.WORKLOADS[wid])
    if sizes is not None:
        wl["sizes"] = sizes
    if dtype is not None and dtype != wl["dtype"]:
        wl["dtype"] = dtype
        wl["dist"] = {"f32": "uniform", "bf16": "normal", "i32": "int20"}[dtype]
    algo = algo or wl["algo"]
    iters = iters or wl["iters"]
    # reduce-scatter inputs and all-gather outputs are N partitions per rank
    widen = wl["nranks"] if algo in ("reducescatter", "allgather") else 1
    h = A.ar_create(wl["nranks"], max(wl["sizes"]) * widen, A.DTYPES[wl["dtype"]])
    try:
        A.ar_set_option(h, A.AR_OPT_PLACEMENT, placement)
        if group is not None:
            A.ar_set_option(h, A.AR_OPT_GROUP, group)
        if SPLIT is not None:
            A.ar_set_option(h, A.AR_OPT_SPLIT, SPLIT)
        rows = []
        for si, size in enumerate(wl["sizes"]):
            rows.append(bench_size(A, I, h, wid, wl, si, size, algo, iters, warmup, hz,
                                   launch_calls=launch_calls, group=group or 4))
            print(f"# workload {wid} {algo} {wl['dtype']} size {size}: p50 "
                  f"{rows[-1]['p50_us']:.3f} us p99 {rows[-1]['p99_us']:.3f} us",
                  file=sys.stderr, flush=True)
    finally:
        A.ar_destroy(h)
    return wl, algo, iters, rows


def _round_rows(rows):
    return [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
            for r in rows]


def floors(A, placement: int) -> dict:
    """The on-chip floor 2 * L_L2 + L_store: on the nearest XCD pair and position (ar_sol_ex),
    and per rank count on the slowest sender -> receiver XCD pair of the placement."""
    sol = A.ar_sol_ex(placement)
    out = {"sol": sol, "floor_nearest_us": sol["floor_ns"] * 1e-3, "by_nranks": {}}
    for n in (2, 4, 8, 16):
        r = A.ar_sol_ranks(n, placement)
        out["by_nranks"][n] = {
            "store_half_rtt_worst_ns": r["store_half_rtt_worst_ns"],
            "store_half_rtt_best_ns": r["store_half_rtt_best_ns"],
            "worst_pair_xcc": [r["worst_sender_xcc"], r["worst_receiver_xcc"]],
            "floor_us": (2 * sol["l2_load_ns"] + r["store_half_rtt_worst_ns"]) * 1e-3,
        }
    return out


def run_config(A, I, wid: int, steps, warmup: int, hz: float, placement: int, fl: dict,
               copy_gbps: float, algos=None) -> dict:
    names, extra_dtypes = CONFIGS[wid]
    wl0 = I.WORKLOADS[wid]
    cfg = wl0["name"]
    n = wl0["nranks"]
    floor = fl["by_nranks"][max(2, n)]["floor_us"] if n > 1 else fl["floor_nearest_us"]
    rec = {"workload": wl0["name"], "nranks": n, "algos": {}, "floor_us": floor,
           "floor_nearest_us": fl["floor_nearest_us"]}
    for dtype in [wl0["dtype"]] + extra_dtypes:
        for algo in (algos or names):
            wl, algo, iters, rows = run_workload(A, I, wid, algo, steps, warmup, hz, placement,
                                                 dtype=dtype)
            key = algo if dtype == wl0["dtype"] else f"{algo}:{dtype}"
            ent = {"dtype": dtype, "iters": iters, "p50_us": [round(r["p50_us"], 4) for r in rows],
                   "p99_us": [round(r["p99_us"], 4) for r in rows],
                   "p50_gm_us": _gm([r["p50_us"] for r in rows]),
                   "per_size": _round_rows(rows)}
            tr = measured_traffic(cfg, algo, dtype, n, rows)
            if wid == BANDWIDTH:
                rl = hbm_roofline(rows, copy_gbps)
                rl["traffic"] = tr
                ent["algbw_GBps"] = [round(r["algbw_GBps"], 2) for r in rows]
            else:
                rl = latency_roofline(rows, floor, EXCHANGES.get(algo, 1))
                rl["traffic"] = tr
                rl["hbm"] = hbm_roofline(rows, copy_gbps)
                ent["p50_over_floor"] = [round(r["p50_us"] / floor, 3) for r in rows]
                ent["p50_over_floor_nearest"] = [round(r["p50_us"] / fl["floor_nearest_us"], 3)
                                                 for r in rows]
            ent["roofline"] = rl
            rec["algos"][key] = ent
    return rec


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed iterations per size (default: each configuration's own count)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--configs", default="1,2,3,4,5",
                    help="comma-separated workload ids to measure beside the headline (2)")
    ap.add_argument("--workload", type=int, default=None, choices=sorted(range(1, 9)),
                    help="measure this workload alone (with --algo) instead of the configurations")
    ap.add_argument("--algo", default=None)
    ap.add_argument("--dtype", default=None, help="with --workload: override the dtype")
    ap.add_argument("--group", type=int, default=None,
                    help="with --workload: ranks per group of the deterministic LL128 variant")
    ap.add_argument("--placement", type=int, default=0, help="0 XCD per rank, 1 same XCD")
    ap.add_argument("--split", type=int, default=None, choices=(0, 1),
                    help="peer-split one-pass kernels on (1) or off (0) [library default: on]")
    ap.add_argument("--all", action="store_true", help="also run the standalone collectives")
    ap.add_argument("--auto-sweep", action="store_true",
                    help="only measure the crossovers behind AR_ALGO_AUTO (every dtype)")
    ap.add_argument("--scratch-sweep", action="store_true",
                    help="only measure latency versus scratch size (AR_SCRATCH_* caps)")
    ap.add_argument("--sweep-caps", default=None,
                    help="with --scratch-sweep: comma-separated caps in MiB")
    ap.add_argument("--sweep-only", default=None,
                    help="with --scratch-sweep: AR_SCRATCH_ONESHOT or AR_SCRATCH_TWOSHOT only")
    ap.add_argument("--report", default=None, help="write the full report (JSON) here")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sizes", default=None,
                    help="comma-separated message sizes in bytes (with --workload)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run the streaming copy kernel over MIB MiB (5 times) and exit; "
                         "its known byte count scales rocprof FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    global SPLIT
    SPLIT = args.split
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
    if args.scratch_sweep:
        caps = ([int(float(x) * (1 << 20)) for x in args.sweep_caps.split(",")]
                if args.sweep_caps else None)
        rows = scratch_sweep(A, I, hz, args.warmup, args.placement, caps=caps,
                             only=args.sweep_only)
        print(json.dumps({"scratch_sweep": rows}), flush=True)
        return 0
    fl = floors(A, args.placement)
    print(f"# floors {json.dumps(fl)}", file=sys.stderr, flush=True)
    peak = copy_peak(A)
    print(f"# streaming copy {peak['GBps']:.0f} GB/s", file=sys.stderr, flush=True)

    if args.workload is not None:
        sizes = [int(x) for x in args.sizes.split(",")] if args.sizes else None
        wl, algo, iters, rows = run_workload(A, I, args.workload, args.algo, args.steps,
                                             args.warmup, hz, args.placement, sizes,
                                             dtype=args.dtype, group=args.group)
        print(json.dumps({"workload": args.workload, "algo": algo, "dtype": wl["dtype"],
                          "per_size": _round_rows(rows)}), flush=True)
        return 0

    # the headline workload, then every other one
    wanted = [int(c) for c in args.configs.split(",") if c]
    hname = I.WORKLOADS[HEADLINE]["name"]
    configs = {hname: run_config(A, I, HEADLINE, args.steps, args.warmup, hz, args.placement, fl,
                                 peak["GBps"])}
    for wid in wanted:
        if wid != HEADLINE:
            configs[I.WORKLOADS[wid]["name"]] = run_config(A, I, wid, args.steps, args.warmup, hz,
                                                           args.placement, fl, peak["GBps"])
    head = configs[hname]["algos"]["oneshot_sentinel"]
    rows = head["per_size"]
    wl = I.WORKLOADS[HEADLINE]
    iters = head["iters"]
    value = head["p50_gm_us"]
    # one step = one AllReduce of every size of every configuration measured
    total_ms = sum(r["launch_ms"] for c in configs.values() for e in c["algos"].values()
                   for r in e["per_size"])
    roof = dict(head["roofline"])
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "us",
        "n_gpus": 1,
        "steps": iters,
        "warmup": args.warmup,
        "ms_per_step": total_ms / iters,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic",
        "config": {
            "workload": (f"{wl['nranks']} emulated ranks on one MI355X, {wl['dtype']} sum "
                         f"(fp32 accumulation), oneshot_sentinel with double buffering, "
                         f"{min(wl['sizes'])}-{max(wl['sizes'])} bytes per rank (powers of two), "
                         f"{iters} back-to-back iterations per size, fresh inputs per iteration"),
            "nranks": wl["nranks"],
            "algo": "oneshot_sentinel",
            "placement": ["rank per XCD", "all ranks on one XCD"][args.placement],
            "sizes_bytes": wl["sizes"],
        },
        "value_definition": ("geometric mean over the headline workload's message sizes of the "
                             "per-size p50 latency (device wall clock, last rank in to last rank "
                             "out)"),
        "latency_floor": {
            "floor_us": configs[hname]["floor_us"],
            "floor_nearest_us": fl["floor_nearest_us"],
            "formula": ("2*L_L2 + L_store (dependent-load L2 latency; store->poll half round "
                        "trip); floor_us on the slowest XCD pair of the 4-rank placement, "
                        "floor_nearest_us on XCDs 0-1 at their nearest memory position"),
            "l2_load_ns": fl["sol"]["l2_load_ns"],
            "store_half_rtt_ns": fl["sol"]["store_half_rtt_ns"],
            "fence_ns": fl["sol"]["fence_ns"],
            "by_nranks": fl["by_nranks"],
            "p50_smallest_over_floor": head["p50_us"][0] / configs[hname]["floor_us"],
            "p50_smallest_over_floor_nearest": head["p50_us"][0] / fl["floor_nearest_us"],
        },
        "roofline": roof,
        "barrier_baseline": {
            "algo": "barrier2",
            "value": configs[hname]["algos"]["barrier2"]["p50_gm_us"],
            "unit": "us",
            "p50_us": configs[hname]["algos"]["barrier2"]["p50_us"],
        },
        "configs": {c: _summary(rec) for c, rec in configs.items()},
        "copy_peak_GBps": peak["GBps"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(I, HEADLINE, wl)
        # at most 16 host threads, whatever os.cpu_count() reports
        line["cpu_baseline"]["multi_thread"] = cpu_baseline_threads(
            I, HEADLINE, wl, max(1, min(16, os.cpu_count() or 1)))
    report = {"main": line, "configs": configs, "floors": fl}
    if args.all:
        report["collectives"] = run_collectives(A, I, hz, args.warmup, args.placement)
    if args.report:
        with open(args.report, "w") as f:
            json.dump(report, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


def _summary(rec: dict) -> dict:
    """A configuration's record for the JSON line: per algorithm the per-size p50 / p99, the
    roofline and (latency configurations) p50 over the floor; the full per-size records go to
    --report."""
    out = {"workload": rec["workload"], "nranks": rec["nranks"], "floor_us": rec["floor_us"],
           "floor_nearest_us": rec["floor_nearest_us"], "algos": {}}
    for k, e in rec["algos"].items():
        s = {kk: e[kk] for kk in ("dtype", "iters", "p50_us", "p99_us", "p50_gm_us",
                                  "p50_over_floor", "algbw_GBps") if kk in e}
        s["sizes_bytes"] = [r["bytes"] for r in e["per_size"]]
        s["kernels"] = sorted({r["launch"]["kernel"] for r in e["per_size"]})
        rl = dict(e["roofline"])
        rl.pop("bound_us", None)
        s["roofline"] = rl
        out["algos"][k] = s
    return out


def auto_sweep(A, I, hz, warmup, placement, iters=100):
    """p50 of the candidate kernels for N in {2,3,4,8,16} and per-rank sizes 128 B .. 2 MiB, for
    every dtype: the measurements behind the automatic algorithm choice (AR_ALGO_AUTO). The
    LL128-style kernel is a candidate for fp32 and int32."""
    sizes = [128 << (2 * k) for k in range(7)] + [2 << 20]
    dists = {"f32": "uniform", "bf16": "normal", "i32": "int20"}
    out = []
    for dtype in ("f32", "bf16", "i32"):
        algos = ["oneshot_ll", "oneshot_sentinel", "twoshot"]
        if dtype != "bf16":
            algos.append("ll128_atomic")
        for n in (2, 3, 4, 8, 16):
            wl = dict(nranks=n, dtype=dtype, dist=dists[dtype], sigma=1.0, sizes=sizes)
            h = A.ar_create(n, max(sizes), A.DTYPES[dtype])
            try:
                A.ar_set_option(h, A.AR_OPT_PLACEMENT, placement)
                for si, size in enumerate(sizes):
                    row = {"dtype": dtype, "nranks": n, "bytes": size}
                    for algo in algos:
                        r = bench_size(A, I, h, 6, wl, si, size, algo, iters, warmup, hz,
                                       launch_calls=0)
                        row[algo] = round(r["p50_us"], 3)
                    row["best"] = min(algos, key=lambda a: row[a])
                    print(f"# sweep {json.dumps(row)}", file=sys.stderr, flush=True)
                    out.append(row)
            finally:
                A.ar_destroy(h)
    return out


def scratch_sweep(A, I, hz, warmup, placement, iters=50, caps=None, only=None):
    """Latency (p50) and algBW versus the scratch caps (AR_SCRATCH_ONESHOT / AR_SCRATCH_TWOSHOT,
    bytes per rank per protocol): the MI355X counterpart of the pages' scratch-size sweep. Each
    cap is applied to the protocol it governs; messages larger than a slot run in chunks."""
    caps = caps or [1 << 20, 4 << 20, 16 << 20, 64 << 20, 256 << 20]
    plan = [
        # (cap variable, workload, algo, dtype, sizes)
        ("AR_SCRATCH_ONESHOT", 2, "oneshot_sentinel", "bf16", [1 << 14, 1 << 17, 1 << 18]),
        ("AR_SCRATCH_ONESHOT", 4, "oneshot_sentinel", "f32", [1 << 15, 1 << 18, 1 << 20]),
        ("AR_SCRATCH_TWOSHOT", 3, "twoshot", "bf16", [1 << 17, 1 << 20]),
        ("AR_SCRATCH_TWOSHOT", 4, "ll128_atomic", "f32", [1 << 18, 1 << 22]),
        ("AR_SCRATCH_TWOSHOT", 4, "twoshot", "f32", [1 << 20, 1 << 22]),
        ("AR_SCRATCH_TWOSHOT", 5, "twoshot", "i32", [16 << 20, 64 << 20, 256 << 20]),
        ("AR_SCRATCH_TWOSHOT", 5, "twoshot", "f32", [16 << 20, 256 << 20]),
    ]
    if only:
        plan = [p for p in plan if p[0] == only]
    out = []
    saved = {k: os.environ.get(k) for k in ("AR_SCRATCH_ONESHOT", "AR_SCRATCH_TWOSHOT")}
    try:
        for var, wid, algo, dtype, sizes in plan:
            for cap in caps:
                os.environ[var] = str(cap)
                wl = dict(I.WORKLOADS[wid], dtype=dtype, sizes=sizes,
                          dist={"f32": "uniform", "bf16": "normal", "i32": "int20"}[dtype])
                it = 20 if wid == 5 else iters
                h = A.ar_create(wl["nranks"], max(sizes), A.DTYPES[dtype])
                try:
                    A.ar_set_option(h, A.AR_OPT_PLACEMENT, placement)
                    for si, size in enumerate(sizes):
                        r = bench_size(A, I, h, wid, wl, si, size, algo, it, warmup, hz,
                                       launch_calls=0, check=False)
                        row = {"cap_var": var, "cap_bytes": cap, "workload": wid, "algo": algo,
                               "dtype": dtype, "nranks": wl["nranks"], "bytes": size,
                               "chunks": r["launch"]["chunks"], "p50_us": round(r["p50_us"], 3),
                               "algbw_GBps": round(r["algbw_GBps"], 2),
                               "alg_GBps_event": round(r["alg_GBps_event"], 1)}
                        print(f"# scratch {json.dumps(row)}", file=sys.stderr, flush=True)
                        out.append(row)
                finally:
                    A.ar_destroy(h)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return out


def run_collectives(A, I, hz, warmup, placement):
    out = {}
    for wid in (6, 7, 8):
        wl, algo, iters, rows = run_workload(A, I, wid, None, None, warmup, hz, placement)
        out[f"{wid}:{algo}:{wl['dtype']}"] = _round_rows(rows)
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
