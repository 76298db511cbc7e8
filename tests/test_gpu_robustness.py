"""GPU tests of the protocol edges: int32 sums equal to the sentinel, launches after a timeout,
writes past the end of an output, the optional input check, and where the workgroups of a real
AllReduce grid run (XCC ids read inside the kernel).

Every case runs through the C ABI and compares with the CPU oracle bit for bit (int32) or at the
method's tolerance (the LL128-style fp32 path).
"""

import numpy as np
import pytest

from tests.gpu_util import (ALGO_NAMES, assert_matches, draw, elem_bytes, from_device, handle,
                            oracle_sum, run_allreduce, supports, to_device)

pytestmark = pytest.mark.gpu

INT32_MIN = -(1 << 31)


def _say(*a):
    print(*a, flush=True)


def _sentinel_sums(n: int, count: int, seed: int) -> np.ndarray:
    """int32 inputs (none equal to INT32_MIN) whose rank sums hit INT32_MIN at every third
    element: exactly (n equal parts of -2^31) and by wrap-around (2^31 reached from above);
    the other elements are ordinary draws."""
    x = draw("i32", n, count, seed=seed)
    for i in range(0, count, 3):
        if (i // 3) % 2 == 0:
            # -2^31 split into n equal-ish parts, none of them INT32_MIN
            parts = [-(1 << 31) // n] * n
            parts[0] += -(1 << 31) - sum(parts)
            x[:, i] = parts
        else:
            # 2^31 (one past INT32_MAX) wraps to INT32_MIN
            parts = [(1 << 31) // n] * n
            parts[-1] += (1 << 31) - sum(parts)
            x[:, i] = np.array(parts, dtype=np.int64).astype(np.int32)
    assert not np.any(x == INT32_MIN)
    return x


@pytest.mark.parametrize("algo", ["twoshot", "ll128_atomic", "auto", "oneshot_sentinel"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_int32_sums_equal_to_the_sentinel(n, algo):
    """int32 sums may take every value, INT32_MIN included: the phases that send sums must not
    mistake such a sum for an empty sentinel slot (the call would time out or return stale
    data). Small and large counts, so that AUTO reaches two-shot."""
    for count in (33, 4099, 65536):
        _say(f"case n={n} algo={algo} count={count}")
        x = _sentinel_sums(n, count, seed=n * 100 + count % 97)
        want = oracle_sum(x)
        assert np.sum(want == INT32_MIN) >= count // 3
        with handle(n, count * 4, "i32", timeout_us=500000) as h:
            got = run_allreduce(h, x, algo)
        for r in range(n):
            bad = np.nonzero(got[r] != want)[0]
            assert bad.size == 0, f"rank {r} wrong at {bad[:8]}"


@pytest.mark.parametrize("algo", ["oneshot_sentinel", "twoshot", "ll128_atomic"])
def test_launch_after_a_timeout_writes_nothing(algo):
    """A call enqueued behind a call that timed out (fault forced from the host: rank 1 withholds
    its data) must not read stale scratch as if it were its data: its kernels exit at entry and
    its outputs keep their previous bytes. ar_check then reports the timeout."""
    from latency_collectives_amd import _ar as A
    import torch

    n, count, dtype = 4, 2048, "f32"
    with handle(n, count * 4, dtype, timeout_us=200000) as h:
        x = draw(dtype, n, count, seed=7)
        ins = to_device(x)
        first = [torch.zeros_like(t) for t in ins]
        second = [torch.full_like(t, 0.25) for t in ins]
        A.ar_set_option(h, A.AR_OPT_WITHHOLD_RANK, 1)
        A.ar_allreduce(h, ins, first, count, A.ALGOS[algo])
        A.ar_set_option(h, A.AR_OPT_WITHHOLD_RANK, -1)
        # enqueued while the first launch is still polling (200 ms timeout)
        A.ar_allreduce(h, ins, second, count, A.ALGOS[algo])
        with pytest.raises(A.ArError) as e:
            A.ar_check(h)
        assert e.value.code == A.AR_ETIMEOUT
        for r in range(n):
            assert torch.all(second[r] == 0.25), f"rank {r}: a launch after the timeout wrote"


CANARY_COUNTS = [1, 3, 33, 257]


def _canary_outputs(n: int, count: int, dtype: str):
    """Outputs that are views into larger buffers: 64 bytes of canary before and after each."""
    import torch

    eb = elem_bytes(dtype)
    pad = 64 // eb
    tdt = {"f32": torch.float32, "bf16": torch.int16, "i32": torch.int32}[dtype]
    bufs = [torch.empty(count + 2 * pad, dtype=tdt, device="cuda") for _ in range(n)]
    for b in bufs:
        b.view(torch.uint8).fill_(0xA5)
    return bufs, [b[pad:pad + count] for b in bufs], pad


def _check_canary(bufs, pad, count):
    for r, b in enumerate(bufs):
        raw = b.view(-1).cpu().numpy().view(np.uint8)
        eb = raw.size // b.numel()
        head, tail = raw[:pad * eb], raw[(pad + count) * eb:]
        assert np.all(head == 0xA5) and np.all(tail == 0xA5), f"rank {r} wrote outside its output"


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [2, 3, 8])
def test_outputs_not_overrun(n, dtype):
    """Ragged tails are handled by the buffer unit's range check: the bytes just before and after
    every output stay untouched, for every AllReduce algorithm and the three collectives (odd
    bf16 lengths included)."""
    from latency_collectives_amd import _ar as A
    import torch

    maxc = max(CANARY_COUNTS)
    with handle(n, n * maxc * 16, dtype) as h:
        for algo in ALGO_NAMES:
            if not supports(algo, dtype):
                continue
            for count in CANARY_COUNTS:
                _say(f"case n={n} dtype={dtype} algo={algo} count={count}")
                x = draw(dtype, n, count, seed=count)
                ins = to_device(x)
                bufs, outs, pad = _canary_outputs(n, count, dtype)
                A.ar_allreduce(h, ins, outs, count, A.ALGOS[algo])
                A.ar_check(h)
                _check_canary(bufs, pad, count)
                assert_matches(from_device(outs, x.dtype), x, algo, dtype)
        for op in ("reducescatter", "allgather", "broadcast"):
            eb = elem_bytes(dtype)
            for count in CANARY_COUNTS:
                part = count
                if op in ("reducescatter", "allgather") and (part * eb) % 16:
                    part = (part * eb + 15) // 16 * 16 // eb  # whole 16-byte partitions
                in_count = n * part if op == "reducescatter" else part
                out_count = n * part if op == "allgather" else part
                _say(f"case n={n} dtype={dtype} op={op} count={part}")
                x = draw(dtype, n, in_count, seed=count + 1)
                ins = to_device(x)
                bufs, outs, pad = _canary_outputs(n, out_count, dtype)
                if op == "reducescatter":
                    A.ar_reducescatter(h, ins, outs, part)
                elif op == "allgather":
                    A.ar_allgather(h, ins, outs, part)
                else:
                    A.ar_broadcast(h, ins[0], outs, part, 0)
                A.ar_check(h)
                _check_canary(bufs, pad, out_count)


def test_input_check_names_the_sentinel():
    """AR_OPT_CHECK_INPUTS: an input equal to the sentinel is refused with AR_EINVAL naming the
    first rank and element (nothing is launched); clean inputs pass and reduce correctly."""
    from latency_collectives_amd import _ar as A

    for dtype, bad in (("f32", np.uint32(0xFFFFFFFF)), ("bf16", np.uint16(0xFFFF)),
                       ("i32", np.uint32(0x80000000))):
        n, count = 4, 1001
        with handle(n, count * 4, dtype, check_inputs=1) as h:
            x = draw(dtype, n, count, seed=11)
            got = run_allreduce(h, x, "oneshot_sentinel")
            assert_matches(got, x, "oneshot_sentinel", dtype)
            y = x.copy()
            view = y.view(np.uint16 if dtype == "bf16" else np.uint32)
            view[2, 777] = bad
            view[3, 5] = bad
            before = A.ar_epoch(h)
            with pytest.raises(A.ArError) as e:
                run_allreduce(h, y, "twoshot")
            assert e.value.code == A.AR_EINVAL
            assert "element 777 of rank 2" in str(e.value) and "2 input element" in str(e.value)
            assert A.ar_epoch(h) == before  # nothing was launched
            # the broadcast checks the root's input only
            ins = to_device(y)
            import torch

            outs = [torch.empty_like(t) for t in ins]
            A.ar_broadcast(h, ins[1], outs, count, 1)
            A.ar_check(h)
            with pytest.raises(A.ArError):
                A.ar_broadcast(h, ins[3], outs, count, 3)


@pytest.fixture(scope="module")
def kernel_resources():
    """Code-object metadata of every kernel of the library (register counts, LDS, private
    segment), read from the library file in plain Python."""
    from latency_collectives_amd import build
    from tests import kernel_meta as KM

    return KM.metadata_from_library(build.ensure_built())


def _check_capacity(kernel_resources, plan, dt_id, n, xcc, mapped):
    """The workgroups that wait for one another (the ranks' workgroups) fit at once on the XCDs
    they ran on: per XCD at most (its compute units) x (workgroups per compute unit), counted
    from the kernel's code-object metadata independently of the occupancy query; the query
    gives the same count as the metadata (registers, SGPRs, wave slots and LDS are all it needs
    to count: no kernel has a private segment), and the plan keeps one workgroup per compute
    unit free whenever the query allows more than one."""
    import torch

    from tests import kernel_meta as KM

    nmax = 2 if n <= 2 else 4 if n <= 4 else 8 if n <= 8 else 16
    sym = KM.kernel_symbol(plan["kernel"], dt_id, nmax)
    meta = kernel_resources[sym]
    assert meta[".private_segment_fixed_size"] == 0, sym
    props = torch.cuda.get_device_properties(0)
    max_waves = props.max_threads_per_multi_processor // 64 // KM.SIMDS_PER_CU
    by_meta = KM.workgroups_per_cu(meta, plan["threads"], max_waves)
    upper = KM.workgroups_per_cu(meta, plan["threads"], max_waves, sgpr_rule=False)
    api = plan["resident_per_cu"]
    _say(f"  {sym}: {plan['threads']} threads, occupancy query {api}, from metadata {by_meta} "
         f"(VGPR / wave-slot / LDS bound {upper})")
    assert 1 <= api <= upper, (sym, api, upper)
    assert api == by_meta, (sym, api, by_meta)  # the query counts what the metadata says
    cus_per_xcd = plan["cu_count"] // 8
    planned_per_cu = api - 1 if api > 1 else api
    per_xcc = np.bincount(xcc[mapped].astype(np.int64), minlength=8)
    assert per_xcc.max() <= cus_per_xcd * planned_per_cu, (sym, per_xcc.tolist(), api)
    assert per_xcc.max() <= cus_per_xcd * by_meta


@pytest.mark.parametrize("placement", [0, 1, 2])
@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_launch_record_matches_decode(n, placement, kernel_resources):
    """Every workgroup of a real AllReduce grid records the XCC it ran on and the rank it
    decoded. Dispatch is round-robin over the 8 XCDs (workgroup w on XCD w % 8), every (rank,
    workgroup) pair appears exactly once, each rank sits on the XCDs its placement gives it:
    rank r on XCD r % 8 (and r + N, r + 2N, ... when it spans several), all on XCD 0 for the
    same-XCD placement; and the ranks' workgroups fit on their XCDs at once (counted from the
    kernels' register and LDS use). The cases cover the one-pass, multi-pass and bulk kernels."""
    from latency_collectives_amd import _ar as A

    cases = [(64, "oneshot_sentinel"), (1 << 16, "oneshot_sentinel"), (1 << 18, "twoshot"),
             (1 << 14, "ll128_atomic"), (1 << 12, "ll128_det"), (1 << 12, "barrier2"),
             (1 << 18, "oneshot_ll"), (1 << 20, "oneshot_sentinel"), (1 << 21, "twoshot")]
    for count, algo in cases:
        with handle(n, count * 4, "f32", placement=placement, record_launch=1) as h:
            try:
                plan = A.ar_plan_info(h, count, A.ALGOS[algo])
            except A.ArError as e:  # a shape the placement cannot hold is refused, not launched
                assert e.code == A.AR_ENORES, e
                _say(f"case n={n} placement={placement} {algo} count={count}: refused ({e})")
                continue
            _say(f"case n={n} placement={placement} {algo} count={count} plan={plan}")
            x = draw("f32", n, count, seed=5)
            got = run_allreduce(h, x, algo)
            assert_matches(got, x, algo, "f32")
            rec = A.ar_read_region(h, 0, A.REGION_LAUNCH_RECORD, 4 * plan["grid"]).view(np.uint32)
        xcc = rec & 0xFF
        rank = ((rec >> 8) & 0xFF).astype(np.int64) - 1
        cta = (rec >> 16).astype(np.int64)
        w = np.arange(plan["grid"])
        assert np.all(xcc == w % 8), "dispatch is not round-robin over the XCDs"
        mapped = rank >= 0
        pairs = set(zip(rank[mapped].tolist(), cta[mapped].tolist()))
        assert len(pairs) == mapped.sum() == n * plan["ctas"]
        _check_capacity(kernel_resources, plan, 0, n, xcc, mapped)
        for r in range(n):
            on = set(xcc[rank == r].tolist())
            if placement == 0:
                allowed = {x for x in range(8) if x % n == r} if n < 8 and 8 % n == 0 else {r % 8}
                assert on <= allowed and (r % 8) in on, f"rank {r} on XCDs {on}"
            elif placement == 1:
                assert on == {0}, f"rank {r} on XCDs {on}"


@pytest.mark.parametrize("n", [2, 8, 16])
def test_cooperative_launch(n):
    """AR_OPT_COOPERATIVE: the runtime checks that each grid can be resident at once before it
    starts it. Every planned grid passes the check (one-pass, multi-pass and bulk kernels, the
    standalone collectives too) and the results are unchanged."""
    import time

    import torch

    from latency_collectives_amd import _ar as A

    cases = [(64, "oneshot_ll"), (1000, "oneshot_sentinel"), (1 << 16, "twoshot"),
             (1 << 21, "twoshot"), (4096, "ll128_atomic"), (4096, "ll128_det"),
             (777, "barrier2"), (1 << 20, "oneshot_sentinel")]
    for count, algo in cases:
        _say(f"case n={n} {algo} count={count}")
        x = draw("f32", n, count, seed=count % 97)
        with handle(n, count * 4, "f32", cooperative=1) as h:
            got = run_allreduce(h, x, algo)
            assert_matches(got, x, algo, "f32")
            if count == 1000:
                ins = to_device(x)
                outs = [torch.empty_like(t) for t in ins]
                for coop in (1, 0):
                    A.ar_set_option(h, A.AR_OPT_COOPERATIVE, coop)
                    A.ar_allreduce(h, ins, outs, count, A.AR_ONESHOT_SENTINEL)
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    for _ in range(50):
                        A.ar_allreduce(h, ins, outs, count, A.AR_ONESHOT_SENTINEL)
                    torch.cuda.synchronize()
                    _say(f"  cooperative={coop}: {(time.perf_counter() - t0) / 50 * 1e6:.1f} "
                         "us per call (host, back to back)")
                A.ar_check(h)
                assert_matches(from_device(outs, x.dtype), x, algo, "f32")
    # a standalone collective with the option on
    count = n * 1024  # partitions of whole 16-byte units
    x = draw("bf16", n, count, seed=3)
    with handle(n, count * 2, "bf16", cooperative=1) as h:
        ins = to_device(x)
        outs = [torch.empty((count // n,), dtype=torch.int16, device="cuda") for _ in range(n)]
        A.ar_reducescatter(h, ins, outs, count // n)
        A.ar_check(h)
        got = from_device(outs, x.dtype)
    ref = oracle_sum(x)
    for r in range(n):
        assert np.array_equal(got[r], ref[r * (count // n):(r + 1) * (count // n)])
