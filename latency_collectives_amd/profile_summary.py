"""Summarise rocprofv3 runs of bench.py into profiles/ (measurement tooling, not the product).

    python -m latency_collectives_amd.profile_summary OUT

OUT holds the output of the commands that `commands(OUT)` lists (run on one MI355X from the
repository root, with TMPDIR=/tmp): a kernel trace of the default benchmark, two counter runs of
it (FETCH_SIZE, WRITE_SIZE), the same two counters on the streaming copy of known size, and
bench.py's --report of each benchmark run. Every per-size record of the report names its timed
launch (`dispatch`: the index among the AllReduce kernel launches of the process), so each timed
launch is found in the trace and the counter runs without guessing.

Writes profiles/traffic.json (HBM bytes per AllReduce, per configuration, algorithm, dtype, rank
count and size, with the sha256 of the kernel sources they were taken on; bench.py reports them
only while the sources match) and one profiles/<algorithm>__<workload>.md per workload and
algorithm with the kernel statistics, each timed launch's trace and event durations, and its
algorithmic against its counted bytes.
"""

from __future__ import annotations

import csv
import glob
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
AR_KERNEL = re.compile(r"ar::ar_kernel(_bulk)?<")

TITLES = {
    "oneshot_ll_n2_f32_128B": "2 ranks, fp32, 128 B",
    "oneshot_sentinel_n4_bf16_1K-256K": "4 ranks, bf16, 1 KiB - 256 KiB",
    "twoshot_n8_bf16_tp_decode_8192": ("8 ranks, bf16, [tokens, 8192] for tokens 1..64 "
                                       "(16 KiB - 1 MiB)"),
    "ll128_vs_oneshot_vs_barrier_n16_f32_4K-4M": "16 ranks, fp32, 4 KiB - 4 MiB",
    "twoshot_n8_bandwidth_16M-256M": "8 ranks, int32 and fp32, 16 MiB - 256 MiB",
}


def commands(out: str) -> dict:
    bench = "python3 bench.py --no-cpu-baseline"
    return {
        "trace": (f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/trace -o run -- "
                  f"{bench} --report {out}/trace_report.json"),
        "fetch": (f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/fetch -o run -- "
                  f"{bench} --report {out}/fetch_report.json"),
        "write": (f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/write -o run -- "
                  f"{bench} --report {out}/write_report.json"),
        "copy_fetch": (f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/copy_fetch -o run"
                       " -- python3 bench.py --calibrate-copy 1024"),
        "copy_write": (f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/copy_write -o run"
                       " -- python3 bench.py --calibrate-copy 1024"),
    }


def _one(pattern: str) -> str:
    f = glob.glob(pattern, recursive=True)
    if len(f) != 1:
        raise FileNotFoundError(f"{pattern}: {f}")
    return f[0]


def _rows(path: str) -> list:
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _counter_by_dispatch(run_dir: str) -> dict:
    """Dispatch id -> (kernel name, counter value summed over the dispatch's rows)."""
    d = {}
    for r in _rows(_one(os.path.join(run_dir, "**", "*counter_collection.csv"))):
        did = int(r["Dispatch_Id"])
        name, v = d.get(did, (r["Kernel_Name"], 0.0))
        d[did] = (name, v + float(r["Counter_Value"]))
    return d


def _ar_dispatches(by_id: dict) -> list:
    """The AllReduce kernel launches, in dispatch order: [(dispatch id, name, value)]."""
    return [(i, n, v) for i, (n, v) in sorted(by_id.items()) if AR_KERNEL.search(n)]


def _copy_scale(run_dir: str, nbytes: int = 1 << 30) -> float:
    vals = [v for _, (n, v) in sorted(_counter_by_dispatch(run_dir).items()) if "stream_copy" in n]
    return nbytes / (statistics.median(vals) * 1024.0)


def _records(report: dict):
    """(workload, algo key, dtype, nranks, per-size record) for every timed launch of a report."""
    for wl, rec in report["configs"].items():
        for key, ent in rec["algos"].items():
            algo = key.split(":")[0]
            for r in ent["per_size"]:
                yield wl, algo, ent["dtype"], rec["nranks"], r


def summarise(out: str) -> None:
    from bench import kernel_source_hash  # the same hash bench.py checks

    cmds = commands(out)
    fetch_scale = _copy_scale(os.path.join(out, "copy_fetch"))
    write_scale = _copy_scale(os.path.join(out, "copy_write"))
    reports = {k: json.load(open(os.path.join(out, f"{k}_report.json")))
               for k in ("trace", "fetch", "write")}
    trace = sorted(_rows(_one(os.path.join(out, "trace", "**", "*kernel_trace.csv"))),
                   key=lambda r: int(r["Dispatch_Id"]))
    ar_trace = [r for r in trace if AR_KERNEL.search(r["Kernel_Name"])]
    stats = _rows(_one(os.path.join(out, "trace", "**", "*kernel_stats.csv")))
    fetch = _ar_dispatches(_counter_by_dispatch(os.path.join(out, "fetch")))
    write = _ar_dispatches(_counter_by_dispatch(os.path.join(out, "write")))
    entries, groups = {}, {}
    recs = {k: list(_records(reports[k])) for k in reports}
    for (wl, algo, dt, n, r), (_, _, _, _, rf), (_, _, _, _, rw) in zip(
            recs["trace"], recs["fetch"], recs["write"]):
        assert r["bytes"] == rf["bytes"] == rw["bytes"]
        d = ar_trace[r["dispatch"]]
        _, fname, fkib = fetch[rf["dispatch"]]
        _, wname, wkib = write[rw["dispatch"]]
        assert d["Kernel_Name"] == fname == wname, (d["Kernel_Name"], fname, wname)
        it = r["iters"]
        fb, wb = fkib * 1024.0 * fetch_scale, wkib * 1024.0 * write_scale
        row = {
            "bytes": r["bytes"], "iters": it,
            "trace_ms": (int(d["End_Timestamp"]) - int(d["Start_Timestamp"])) * 1e-6,
            "event_ms": r["launch_ms"], "p50_us": r["p50_us"],
            "kernel": d["Kernel_Name"],
            "alg_bytes_per_ar": r["alg_bytes_per_call"],
            "fetch_bytes_per_ar": fb / rf["iters"], "write_bytes_per_ar": wb / rw["iters"],
        }
        row["hbm_bytes_per_ar"] = row["fetch_bytes_per_ar"] + row["write_bytes_per_ar"]
        key = f"{wl}:{algo}:{dt}:n{n}:{r['bytes']}"
        entries[key] = {k: row[k] for k in ("hbm_bytes_per_ar", "fetch_bytes_per_ar",
                                            "write_bytes_per_ar", "alg_bytes_per_ar", "kernel")}
        groups.setdefault((wl, algo), []).append((dt, row))
    traffic = {
        "source_sha256": kernel_source_hash(),
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "definition": ("HBM bytes per AllReduce = (FETCH_SIZE x fetch_scale + WRITE_SIZE x "
                       "write_scale) x 1024 / iterations of the timed launch; the scales make the "
                       "streaming copy of 1 GiB read and write exactly 1 GiB each"),
        "commands": cmds,
        "entries": entries,
    }
    prof = os.path.join(ROOT, "profiles")
    with open(os.path.join(prof, "traffic.json"), "w") as fh:
        json.dump(traffic, fh, indent=1)
    for (wl, algo), rows in groups.items():
        names = sorted({row["kernel"] for _, row in rows})
        L = [f"# {wl} ({TITLES.get(wl, '')}), {algo}", "",
             "Commands (repository root, one MI355X, ROCm 7.2, `export TMPDIR=/tmp`; OUT is any "
             "directory), then `python -m latency_collectives_amd.profile_summary OUT`:", "",
             "```", *cmds.values(), "```", "",
             "## Kernel statistics of the whole trace run (top 8 by time)", "",
             "| kernel | calls | total ms | average µs | % |", "|---|---|---|---|---|"]
        for srow in sorted(stats, key=lambda x: -float(x["TotalDurationNs"]))[:8]:
            nm = srow["Name"] if len(srow["Name"]) <= 80 else srow["Name"][:80]
            L.append(f"| `{nm}` | {srow['Calls']} | {float(srow['TotalDurationNs']) * 1e-6:.3f} | "
                     f"{float(srow['AverageNs']) * 1e-3:.2f} | {float(srow['Percentage']):.2f} |")
        L += ["", f"## Timed launches ({', '.join('`' + n + '`' for n in names)})", "",
              "One launch per message size runs `iters` AllReduces back to back. `trace` is "
              "rocprofv3's kernel duration, `event` the HIP-event time bench.py measured on the "
              "launch stream in the trace run. Bytes are per AllReduce (all ranks): `alg` counts "
              "every logical read and write once (ar_alg_bytes), `HBM` = FETCH_SIZE x "
              f"{fetch_scale:.4f} + WRITE_SIZE x {write_scale:.4f} (KiB x 1024; factors from the "
              "streaming copy of 1 GiB). The counters count L2 misses to the memory side (MALL or "
              "HBM).", "",
              "| dtype | bytes/rank | iters | p50 µs | trace ms | event ms | alg B/AR | HBM B/AR "
              "| HBM / alg |",
              "|---|---|---|---|---|---|---|---|---|"]
        for dt, row in rows:
            L.append(f"| {dt} | {row['bytes']} | {row['iters']} | {row['p50_us']:.3f} | "
                     f"{row['trace_ms']:.4f} | {row['event_ms']:.4f} | "
                     f"{row['alg_bytes_per_ar']:.4g} | {row['hbm_bytes_per_ar']:.4g} | "
                     f"{row['hbm_bytes_per_ar'] / row['alg_bytes_per_ar']:.3f} |")
        mt = statistics.mean(row["trace_ms"] for _, row in rows)
        me = statistics.mean(row["event_ms"] for _, row in rows)
        L += ["", f"Mean over the timed launches: trace {mt:.4f} ms, event {me:.4f} ms.", ""]
        with open(os.path.join(prof, f"{algo}__{wl}.md"), "w") as fh:
            fh.write("\n".join(L))
        print(f"{wl} {algo}: {len(rows)} launches, kernels {names}")


if __name__ == "__main__":
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    if len(sys.argv) != 2:
        sys.exit("usage: python -m latency_collectives_amd.profile_summary OUT")
    summarise(sys.argv[1])
