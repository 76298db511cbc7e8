"""Host logic of bench.py (CPU only): the roofline arithmetic, the counter-traffic table behind
`roofline.traffic`, and the refusal of more than one GPU."""

import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as B

    return B


def _rows():
    return [{"bytes": 1024, "p50_us": 1.0, "alg_bytes_per_call": 8.0e6, "iters": 10,
             "launch_ms": 0.02, "alg_GBps_event": 4000.0},
            {"bytes": 4096, "p50_us": 4.0, "alg_bytes_per_call": 32.0e6, "iters": 10,
             "launch_ms": 0.08, "alg_GBps_event": 4000.0}]


def test_latency_roofline_bounds(bench):
    rows = _rows()
    one = bench.latency_roofline(rows, 0.5)
    two = bench.latency_roofline(rows, 0.5, exchanges=2)
    # bound = exchanges * floor + bytes / 8 TB/s (8e6 B -> 1 us, 32e6 B -> 4 us)
    assert one["bound_us"] == [1.5, 4.5] and two["bound_us"] == [2.0, 5.0]
    assert math.isclose(one["frac"], math.sqrt((1.5 / 1.0) * (4.5 / 4.0)))
    assert math.isclose(one["achieved"], 2.0) and math.isclose(one["peak"], math.sqrt(1.5 * 4.5))
    assert one["p50_over_bound"] == [round(1 / 1.5, 3), round(4 / 4.5, 3)]
    assert bench.EXCHANGES["twoshot"] == 2 and bench.EXCHANGES["oneshot_sentinel"] == 1


def test_hbm_roofline(bench):
    rl = bench.hbm_roofline(_rows(), 5000.0)
    # (8e6 + 32e6) * 10 bytes in 0.1 ms
    assert math.isclose(rl["achieved"], 4.0e8 / 1e-4 / 1e9)
    assert math.isclose(rl["frac"], rl["achieved"] / 8000.0)
    assert math.isclose(rl["frac_of_copy_peak"], rl["achieved"] / 5000.0)


def test_traffic_table_covers_every_timed_launch(bench):
    """profiles/traffic.json holds a counter record for every (workload, algorithm, dtype,
    size) the default run times, taken on the current kernel sources (otherwise bench.py would
    report `traffic` as null)."""
    from latency_collectives_amd import inputs as I

    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert rec["source_sha256"] == bench.kernel_source_hash(), \
        "kernel sources changed since the counters were taken: re-run the profiling commands"
    for wid, (algos, extra) in bench.CONFIGS.items():
        wl = I.WORKLOADS[wid]
        for dtype in [wl["dtype"]] + extra:
            for algo in algos:
                for size in wl["sizes"]:
                    key = bench.traffic_key(wl["name"], algo, dtype, wl["nranks"], size)
                    e = rec["entries"].get(key)
                    assert e is not None, key
                    # counted bytes are at least the algorithmic ones minus what the L2 absorbs
                    assert e["hbm_bytes_per_ar"] > 0.5 * e["alg_bytes_per_ar"], key
    assert 0.5 < rec["fetch_scale"] < 4 and 0.5 < rec["write_scale"] < 4


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr)
