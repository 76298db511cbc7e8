"""GPU parity: every algorithm, through the C ABI, against the CPU oracle.

Bar: int32 and fixed-rank-order fp32 / bf16 bit-exact; the LL128-style atomic fp32 path within
N * 2^-23 * sum_r |x_r| per element, and bit-exact on dyadic inputs whose partial sums are exact
in any order.
"""

import numpy as np
import pytest

from tests.gpu_util import (ALGO_NAMES, assert_matches, draw, elem_bytes, from_device, handle,
                            run_allreduce, supports, to_device)

pytestmark = pytest.mark.gpu

COUNTS = [1, 3, 8, 33, 257, 1000, 4099, 70001]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
def test_all_algorithms_ragged_counts(n, dtype):
    maxc = max(COUNTS)
    with handle(n, maxc * elem_bytes(dtype), dtype) as h:
        for algo in ALGO_NAMES:
            if not supports(algo, dtype):
                continue
            for i, count in enumerate(COUNTS):
                _say(f"case n={n} dtype={dtype} algo={algo} count={count}")
                x = draw(dtype, n, count, seed=1000 * n + i)
                got = run_allreduce(h, x, algo)
                assert_matches(got, x, algo, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_sentinel_kernels_both_unit_widths(n, dtype):
    """The one-pass sentinel kernels (one-shot and two-shot) with 8-byte units (the default where
    they fit) and with 16-byte units (AR_OPT_NARROW = 0): both match the oracle, ragged counts
    included, and give bit-identical outputs."""
    maxc = max(COUNTS)
    outs = {}
    for narrow in (1, 0):
        with handle(n, maxc * elem_bytes(dtype), dtype, narrow=narrow) as h:
            for algo in ("oneshot_sentinel", "twoshot"):
                for i, count in enumerate(COUNTS):
                    _say(f"case n={n} dtype={dtype} algo={algo} narrow={narrow} count={count}")
                    x = draw(dtype, n, count, seed=3000 * n + i)
                    got = run_allreduce(h, x, algo)
                    assert_matches(got, x, algo, dtype)
                    outs[(narrow, algo, count)] = got
    for (narrow, algo, count), got in outs.items():
        if narrow == 1:
            assert np.array_equal(got.view(np.uint8), outs[(0, algo, count)].view(np.uint8)), \
                f"{algo} count={count}: 8-byte and 16-byte units differ"


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
def test_auto_selection_matches_oracle(dtype):
    """AR_ALGO_AUTO over rank counts and sizes that select each of its kernels, for every dtype.
    fp32 and bf16 must stay bit-exact with the rank-order oracle (AUTO only picks fixed-order
    kernels for floats: never an LL128-style one); int32 may also pick the LL128-style kernel
    (an exact integer sum) and is bit-exact as well."""
    from latency_collectives_amd import _ar as A

    # LL, sentinel, two-shot and their internal kernels (multi-pass, narrow, bulk, peer-split)
    fixed = {1, 2, 3, 7, 8, 9, 10, 11, 26, 27, 28, 29, 33, 34}
    seen = set()
    eb = elem_bytes(dtype)
    for n in (2, 3, 4, 6, 8, 16):
        for nbytes in (128, 2800, 20000, 160000, 600000, 3 << 20):
            count = nbytes // eb
            with handle(n, count * eb, dtype) as h:
                plan = A.ar_plan_info(h, count, A.AR_ALGO_AUTO)
                seen.add(plan["kernel"])
                if dtype != "i32":
                    assert plan["kernel"] in fixed, plan
                x = draw(dtype, n, count, seed=n * 7 + count % 97)
                got = run_allreduce(h, x, "auto")
                assert_matches(got, x, "oneshot_ll", dtype)
    _say(f"auto {dtype}: kernel families {sorted(seen)}")
    assert len(seen) >= 3


@pytest.mark.parametrize("algo", ALGO_NAMES)
def test_in_place(algo):
    n, dtype, count = 4, "f32", 5000
    with handle(n, count * 4, dtype) as h:
        x = draw(dtype, n, count, seed=7)
        got = run_allreduce(h, x, algo, inplace=True)
        assert_matches(got, x, algo, dtype)


@pytest.mark.parametrize("algo", ALGO_NAMES)
def test_chunked_scratch(algo):
    """Scratch capped far below the message: the call runs as many equal chunks, each a step with
    its own sequence number and alternating buffer (double-buffer credits inside one call)."""
    n, count = 4, 100003
    for dtype in ("f32", "i32"):
        env = {"AR_SCRATCH_ONESHOT": 64 << 10, "AR_SCRATCH_TWOSHOT": 64 << 10}
        with handle(n, count * 4, dtype, env=env) as h:
            _say(f"case chunked algo={algo} dtype={dtype}")
            x = draw(dtype, n, count, seed=11)
            got = run_allreduce(h, x, algo)
            assert_matches(got, x, algo, dtype)


def test_ll128_dyadic_exact():
    """Dyadic inputs k * 2^-10: every partial sum is exact, so the atomic path must equal the
    oracle bit for bit whatever order the additions happened in."""
    for n in (2, 8, 16):
        count = 20000
        with handle(n, count * 4, "f32") as h:
            x = draw("f32", n, count, seed=n, dist="dyadic")
            got = run_allreduce(h, x, "ll128_atomic")
            from tests.gpu_util import oracle_sum

            want = oracle_sum(x)
            assert np.array_equal(got[0].view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("algo", ALGO_NAMES)
def test_rank_constant_invariant(algo):
    """Rank r filled with r: every output is N(N-1)/2."""
    for n in (2, 8, 16):
        count = 3001
        with handle(n, count * 4, "f32") as h:
            x = draw("f32", n, count, seed=0, dist="rankconst")
            got = run_allreduce(h, x, algo)
            assert np.all(got == n * (n - 1) // 2)


@pytest.mark.parametrize("narrow", [1, 0])
@pytest.mark.parametrize("algo", ["oneshot_sentinel", "twoshot", "ll128_atomic"])
def test_scratch_rearmed_after_call(algo, narrow):
    """After a call every sentinel slot holds the sentinel again and the atomic destination and
    arrival counters are back to zero: for a message that uses the regular regions and, at
    1000 elements, for one that uses the near regions; with 8- and 16-byte units."""
    from latency_collectives_amd import _ar as A

    n, dtype, count = 4, "f32", 7777
    with handle(n, count * 4, dtype, narrow=narrow) as h:
        for it in range(3):
            for c in (count, 1000):
                x = draw(dtype, n, c, seed=50 + it)
                got = run_allreduce(h, x, algo)
                assert_matches(got, x, algo, dtype)
        for r in range(n):
            for reg in (A.REGION_P1, A.REGION_P2, A.REGION_P1_NEAR, A.REGION_P2_NEAR):
                w = A.ar_read_region(h, r, reg).view(np.uint32)
                assert np.all(w == 0xFFFFFFFF), f"rank {r} region {reg} not re-armed"
            for reg in (A.REGION_ACC, A.REGION_CNT):
                w = A.ar_read_region(h, r, reg).view(np.uint32)
                assert np.all(w == 0), f"rank {r} region {reg} not cleared"


def test_count_zero_and_epoch():
    from latency_collectives_amd import _ar as A

    with handle(2, 1024, "f32") as h:
        e0 = A.ar_epoch(h)
        import torch

        t = [torch.zeros(4, device="cuda"), torch.zeros(4, device="cuda")]
        A.ar_allreduce(h, t, t, 0, A.AR_ONESHOT_LL)
        assert A.ar_epoch(h) == e0 + 1
        A.ar_check(h)


def test_argument_errors_on_device():
    from latency_collectives_amd import _ar as A
    import torch

    with handle(2, 1024, "f32") as h:
        a = [torch.zeros(300, device="cuda") for _ in range(2)]
        with pytest.raises(A.ArError) as e:
            A.ar_allreduce(h, a, a, 300, A.AR_ONESHOT_LL)  # 1200 bytes > max_bytes
        assert e.value.code == A.AR_ETOOBIG
        b = [torch.zeros(64, device="cuda") for _ in range(2)]
        with pytest.raises(A.ArError) as e:
            A.ar_allreduce(h, b, [b[0], b[0]], 64, A.AR_ONESHOT_LL)
        assert e.value.code == A.AR_EINVAL
    with handle(2, 1024, "f32", group=2) as h:
        with pytest.raises(A.ArError) as e:
            A.ar_set_option(h, A.AR_OPT_GROUP, 1)  # a group of one rank is the two-shot
        assert e.value.code == A.AR_EINVAL


@pytest.mark.parametrize("algo", ALGO_NAMES)
def test_withheld_rank_times_out_without_hang(algo):
    """Fault injection forced from the host: rank 1 sends nothing, its peers' bounded polls give
    up after 20 ms, ar_check reports AR_ETIMEOUT, and the handle stays poisoned."""
    from latency_collectives_amd import _ar as A
    import torch

    n, count = 4, 4096
    dtype = "f32"
    with handle(n, count * 4, dtype, timeout_us=20000, withhold_rank=1) as h:
        x = draw(dtype, n, count, seed=3)
        ins = to_device(x)
        outs = [torch.empty_like(t) for t in ins]
        A.ar_allreduce(h, ins, outs, count, A.ALGOS[algo])
        with pytest.raises(A.ArError) as e:
            A.ar_check(h)
        assert e.value.code == A.AR_ETIMEOUT
        assert "timed out" in str(e.value)
        with pytest.raises(A.ArError) as e:
            A.ar_allreduce(h, ins, outs, count, A.ALGOS[algo])
        assert e.value.code == A.AR_ETIMEOUT


@pytest.mark.parametrize("algo", ALGO_NAMES)
@pytest.mark.parametrize("drift", [0, 3])
def test_persistent_loop_every_iteration(algo, drift):
    """ar_bench: many AllReduces in one launch with fresh inputs per iteration; every
    iteration's output is checked (double-buffer credits across iterations, optionally with a
    random per-rank delay before each iteration)."""
    from latency_collectives_amd import _ar as A

    n, dtype, count, iters = 4, "f32", 1500, 60
    with handle(n, count * 4, dtype, drift=drift) as h:
        xs = [draw(dtype, n, count, seed=200 + k) for k in range(iters)]
        ins, outs = [], []
        import torch

        for x in xs:
            d = to_device(x)
            ins += d
            outs += [torch.empty_like(t) for t in d]
        ts, te, ms = A.ar_bench_ex(h, ins, outs, iters, count, A.ALGOS[algo], iters)
        assert ms > 0
        for k in range(iters):
            got = from_device(outs[k * n:(k + 1) * n], np.float32)
            assert_matches(got, xs[k], algo, dtype)
        assert np.all(te.reshape(iters, n) >= ts.reshape(iters, n))


def test_c1_shape_1000_iterations_all_checked():
    """2 ranks, fp32, 32 elements, one-shot LL, 1000 back-to-back iterations with fresh inputs;
    all 1000 outputs checked bit for bit."""
    from latency_collectives_amd import _ar as A
    import torch

    n, count, iters = 2, 32, 1000
    with handle(n, 128, "f32") as h:
        xs = [draw("f32", n, count, seed=k) for k in range(iters)]
        # evenly spaced sets (one [iters, count] buffer per rank): the table-free path
        big = [torch.from_numpy(np.stack([xs[k][r] for k in range(iters)])).cuda()
               for r in range(n)]
        obig = [torch.empty_like(b) for b in big]
        ins = [big[r][k] for k in range(iters) for r in range(n)]
        outs = [obig[r][k] for k in range(iters) for r in range(n)]
        A.ar_bench(h, ins, outs, iters, count, A.AR_ONESHOT_LL, iters)
        for k in range(iters):
            got = np.stack([obig[r][k].cpu().numpy() for r in range(n)])
            assert_matches(got, xs[k], "oneshot_ll", "f32")


@pytest.mark.parametrize("placement", [0, 1, 2])
def test_placements(placement):
    n, dtype, count = 8, "bf16", 9000
    with handle(n, count * 2, dtype, placement=placement) as h:
        for algo in ("oneshot_ll", "oneshot_sentinel", "twoshot"):
            x = draw(dtype, n, count, seed=placement)
            got = run_allreduce(h, x, algo)
            assert_matches(got, x, algo, dtype)


def test_sol_microbench_sane():
    from latency_collectives_amd import _ar as A

    x = A.ar_sol_ex(A.AR_PLACE_XCD)
    _say("sol xcd", x)
    assert x["l2_load_ns"] > 0 and x["store_half_rtt_ns"] > 0 and x["fence_ns"] > 0
    assert x["xcc_a"] != x["xcc_b"]
    s = A.ar_sol_ex(A.AR_PLACE_SAME)
    _say("sol same", s)
    assert s["xcc_a"] == s["xcc_b"]
    assert x["floor_ns"] == pytest.approx(2 * x["l2_load_ns"] + x["store_half_rtt_ns"])
    # the floor's store term is the line homed near the pair; the other half's is reported too
    assert x["store_half_rtt_far_ns"] >= x["store_half_rtt_ns"] > 0
    # sanity pins of the bound's terms: a store seen from another XCD is no faster than one seen
    # on the same XCD, and a dependent L2 hit is no slower than a store plus release fence
    assert x["store_half_rtt_ns"] >= s["store_half_rtt_ns"]
    assert x["l2_load_ns"] <= x["fence_ns"]
    # the three-value form returns the same terms
    b = A.ar_sol(A.AR_PLACE_XCD)
    assert set(b) == {"fence_ns", "l2_load_ns", "store_half_rtt_ns"}
    assert all(v > 0 for v in b.values())


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_sol_ranks_floor_covers_every_pair(n):
    """The N-rank store term is the slowest (sender, receiver) XCD pair of the placement: at
    least the nearest pair's, and it names two XCDs that hold ranks."""
    from latency_collectives_amd import _ar as A

    near = A.ar_sol_ex(A.AR_PLACE_XCD)
    r = A.ar_sol_ranks(n, A.AR_PLACE_XCD)
    _say(f"sol ranks n={n}", r)
    xcds = {q % 8 for q in range(n)}
    assert r["worst_sender_xcc"] in xcds and r["worst_receiver_xcc"] in xcds
    distinct = len(xcds) * (len(xcds) - 1) + (len(xcds) if n > 8 else 0)
    assert r["pairs"] == distinct
    assert r["store_half_rtt_worst_ns"] >= r["store_half_rtt_best_ns"] > 0
    # the nearest 0-1 position is one of the candidates the worst pair is chosen over, up to the
    # run-to-run spread of a ping-pong
    assert r["store_half_rtt_worst_ns"] >= 0.9 * near["store_half_rtt_ns"]


def test_sixteen_byte_lines_not_torn():
    """The LL protocol's 16-byte line must arrive whole; count torn reads across XCDs."""
    from latency_collectives_amd import _ar as A

    for placement in (A.AR_PLACE_XCD, A.AR_PLACE_SAME):
        torn, reads = A.ar_torn_lines(placement, 64, 200000)
        _say(f"torn-line probe placement={placement}: torn={torn} reads={reads}")
        assert reads > 0
        assert torn == 0
