"""GPU parity of the bandwidth-regime two-shot kernel and of every workload at its full size.

The bulk two-shot runs whenever a chunk is wider than one pass of the rank's workgroups. The
first tests force it at small sizes by capping the workgroups per rank, so that ragged tails,
multi-chunk calls, re-arming and the timeout path are all covered where the oracle is quick.
The full-size tests run the workloads' own shapes in the launch configuration the benchmark
uses: the messages are compared element by element with the oracle (which is a plain fold and
finishes these sizes in seconds), and all ranks' outputs with each other.
"""

import numpy as np
import pytest

from tests.gpu_util import (assert_matches, draw, from_device, handle, run_allreduce,
                            to_device)

pytestmark = pytest.mark.gpu

BULK_COUNTS = [4099, 70001, 250007]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_bulk_twoshot_forced(n, dtype):
    """One or three workgroups per rank: every chunk needs several passes."""
    eb = {"f32": 4, "bf16": 2, "i32": 4}[dtype]
    for ctas in (1, 3):
        with handle(n, max(BULK_COUNTS) * eb, dtype, ctas=ctas) as h:
            for i, count in enumerate(BULK_COUNTS):
                _say(f"case bulk n={n} dtype={dtype} ctas={ctas} count={count}")
                x = draw(dtype, n, count, seed=500 + 10 * n + i)
                got = run_allreduce(h, x, "twoshot")
                assert_matches(got, x, "twoshot", dtype)


def test_bulk_twoshot_chunked_and_rearmed():
    """Scratch capped at 64 KiB: many chunks per call, alternating buffers; afterwards every
    sentinel slot holds the sentinel again."""
    from latency_collectives_amd import _ar as A

    n, count = 4, 300007
    env = {"AR_SCRATCH_TWOSHOT": 64 << 10}
    for dtype in ("f32", "bf16", "i32"):
        eb = 2 if dtype == "bf16" else 4
        with handle(n, count * eb, dtype, env=env, ctas=1) as h:
            for it in range(2):
                _say(f"case bulk chunked dtype={dtype} it={it}")
                x = draw(dtype, n, count, seed=77 + it)
                got = run_allreduce(h, x, "twoshot")
                assert_matches(got, x, "twoshot", dtype)
            sentinel = 0x80000000 if dtype == "i32" else 0xFFFFFFFF
            for r in range(n):
                for reg in (A.REGION_P1, A.REGION_P2):
                    w = A.ar_read_region(h, r, reg).view(np.uint32)
                    assert np.all(w == sentinel), f"rank {r} region {reg} not re-armed"


@pytest.mark.parametrize("n", [2, 4, 8])
def test_bulk_twoshot_small_slots_near_sized(n):
    """A message small enough for the near regions but forced onto one workgroup per rank runs
    the bulk two-shot, whose own slots are capped at 8 KiB here: the call must use the regular
    chunking (several chunks), not the near regions' single chunk."""
    from latency_collectives_amd import _ar as A

    count = n * 2000 * 4 + 5  # about 2000 units per partition, more than one 512-unit slot
    env = {"AR_SCRATCH_TWOSHOT": (2 * n * 8) << 10}
    with handle(n, count * 4, "f32", env=env, ctas=1) as h:
        for it in range(3):
            _say(f"case bulk near-sized n={n} it={it}")
            x = draw("f32", n, count, seed=900 + 10 * n + it)
            got = run_allreduce(h, x, "twoshot")
            assert_matches(got, x, "twoshot", "f32")
        S = count * 4
        assert A.ar_alg_bytes(h, count, A.AR_TWOSHOT) == 2 * n * S + 2 * (n - 1) * S, \
            "the bulk two-shot kernel was not the one planned"


def test_bulk_twoshot_withheld_rank_times_out():
    from latency_collectives_amd import _ar as A
    import torch

    n, count = 4, 70001
    with handle(n, count * 4, "f32", ctas=1, timeout_us=20000, withhold_rank=2) as h:
        x = draw("f32", n, count, seed=5)
        ins = to_device(x)
        outs = [torch.empty_like(t) for t in ins]
        A.ar_allreduce(h, ins, outs, count, A.AR_TWOSHOT)
        with pytest.raises(A.ArError) as e:
            A.ar_check(h)
        assert e.value.code == A.AR_ETIMEOUT


@pytest.mark.parametrize("drift", [0, 3])
def test_bulk_twoshot_persistent_loop(drift):
    """Several bulk AllReduces in one persistent launch (completion flags and double-buffer
    credits across iterations), optionally with a random per-rank delay before each iteration."""
    from latency_collectives_amd import _ar as A
    import torch

    n, dtype, count, iters = 8, "bf16", 100001, 6
    with handle(n, count * 2, dtype, ctas=2, drift=drift) as h:
        xs = [draw(dtype, n, count, seed=900 + k) for k in range(iters)]
        ins, outs = [], []
        for x in xs:
            d = to_device(x)
            ins += d
            outs += [torch.empty_like(t) for t in d]
        A.ar_bench(h, ins, outs, iters, count, A.AR_TWOSHOT, iters)
        for k in range(iters):
            got = from_device(outs[k * n:(k + 1) * n], np.uint16)
            assert_matches(got, xs[k], "twoshot", dtype)


@pytest.mark.parametrize("n,dtype", [(16, "f32"), (16, "bf16"), (12, "f32")])
def test_bulk_twoshot_above_the_two_page_slots(n, dtype):
    """More than 8 ranks and over 1 MiB per rank: the fp32 / bf16 two-shot takes the bulk kernel
    (ragged, odd bf16 length), out of place and in place, against the oracle."""
    from latency_collectives_amd import _ar as A

    size = (2 << 20) + 48
    count = size // (2 if dtype == "bf16" else 4)
    if dtype == "bf16":
        count -= 1
    x = draw(dtype, n, count, seed=90 + n)
    with handle(n, size, dtype) as h:
        plan = A.ar_plan_info(h, count, A.AR_TWOSHOT)
        assert plan["kernel"] == 7 and plan["near"] == 0, plan
        assert A.ar_plan_info(h, (1 << 20) // (2 if dtype == "bf16" else 4), A.AR_TWOSHOT)["kernel"] != 7
        got = run_allreduce(h, x, "twoshot")
        assert_matches(got, x, "twoshot", dtype)
        got_in = run_allreduce(h, x, "twoshot", inplace=True)
        assert np.array_equal(got.view(np.uint8), got_in.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "i32"])
def test_bulk_twoshot_in_place(dtype):
    """In place (output = input): the owners store the all-gather straight into every rank's
    buffer, which is also that rank's input; each owner does so only after all its peers' input
    partitions have reached it, so no input is overwritten before it was sent."""
    from latency_collectives_amd import _ar as A

    n, count = 8, 250007
    x = draw(dtype, n, count, seed=77)
    with handle(n, count * 4, dtype, ctas=2) as h:
        got = run_allreduce(h, x, "twoshot", inplace=True)
    assert_matches(got, x, "twoshot", dtype)


def test_bulk_twoshot_persistent_in_place_loop():
    """A persistent in-place loop on one set (each iteration reduces the previous result): the
    outputs overlap the inputs, so the launch keeps the all-gather in the slots; after k
    iterations every element is N^(k-1) times the first sum (wrapping int32)."""
    from latency_collectives_amd import _ar as A
    import torch

    n, count, iters = 8, 70001, 3
    x = draw("i32", n, count, seed=78)
    with handle(n, count * 4, "i32", ctas=2) as h:
        bufs = to_device(x)
        A.ar_bench(h, bufs, bufs, 1, count, A.AR_TWOSHOT, iters)
        got = from_device(bufs, np.int32)
    first = x.astype(np.int64).sum(axis=0)
    want = ((first * n ** (iters - 1) + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int32)
    for r in range(n):
        assert np.array_equal(got[r], want), f"rank {r}"


# ------------------------------------------------------------------ full workload sizes


def _bench_sets(h, xs, algo, dtype, iters=None):
    """Run the sets xs[k] ([N, count] each) through one persistent launch of `iters` AllReduces
    (default two per set), as the benchmark does (evenly spaced sets of one buffer per rank),
    and check every set."""
    from latency_collectives_amd import _ar as A
    import torch

    n, count = xs[0].shape
    view = np.int16 if dtype == "bf16" else xs[0].dtype
    big = [torch.from_numpy(np.ascontiguousarray(np.stack([x[r] for x in xs]).view(view))).cuda()
           for r in range(n)]
    obig = [torch.empty_like(b) for b in big]
    ins = [big[r][k] for k in range(len(xs)) for r in range(n)]
    outs = [obig[r][k] for k in range(len(xs)) for r in range(n)]
    A.ar_bench(h, ins, outs, len(xs), count, A.ALGOS[algo], iters or 2 * len(xs))
    for k, x in enumerate(xs):
        got = np.stack([obig[r][k].cpu().numpy().view(x.dtype) for r in range(n)])
        assert_matches(got, x, algo, dtype)


def test_full_size_c2_oneshot_sentinel():
    """4 ranks, bf16 normal(0,1), 1 KiB .. 256 KiB per rank."""
    from latency_collectives_amd import inputs as I

    wl = I.WORKLOADS[2]
    with handle(4, max(wl["sizes"]), "bf16") as h:
        for si, size in enumerate(wl["sizes"]):
            _say(f"case c2 size={size}")
            xs = [I.rank_inputs("normal", "bf16", 4, size // 2, 2, si, k) for k in range(3)]
            _bench_sets(h, xs, "oneshot_sentinel", "bf16")


def test_c2_persistent_loop_at_full_iteration_count():
    """The headline configuration's 200 back-to-back iterations in one launch (40 fresh input
    sets, each used five times), every set's output checked, at the smallest, a middle and the
    largest size."""
    from latency_collectives_amd import inputs as I

    with handle(4, 1 << 18, "bf16") as h:
        for si, size in ((0, 1 << 10), (4, 1 << 14), (8, 1 << 18)):
            _say(f"case c2 200 iterations size={size}")
            xs = [I.rank_inputs("normal", "bf16", 4, size // 2, 2, si, k) for k in range(40)]
            _bench_sets(h, xs, "oneshot_sentinel", "bf16", iters=200)


def test_c3_persistent_loop_at_full_iteration_count():
    """The decode configuration's 100 back-to-back two-shot iterations (20 fresh sets, each used
    five times), every set checked, at 1, 8 and 64 tokens."""
    from latency_collectives_amd import inputs as I

    with handle(8, 64 * 8192 * 2, "bf16") as h:
        for si, tokens in ((0, 1), (3, 8), (6, 64)):
            size = tokens * 8192 * 2
            _say(f"case c3 100 iterations tokens={tokens}")
            xs = [I.rank_inputs("normal", "bf16", 8, size // 2, 3, si, k, 0.5) for k in range(20)]
            _bench_sets(h, xs, "twoshot", "bf16", iters=100)


def test_full_size_c3_twoshot():
    """8 ranks, bf16 normal(0,0.5), [tokens, 8192] for tokens 1..64 (16 KiB .. 1 MiB)."""
    from latency_collectives_amd import inputs as I

    wl = I.WORKLOADS[3]
    with handle(8, max(wl["sizes"]), "bf16") as h:
        for si, size in enumerate(wl["sizes"]):
            _say(f"case c3 size={size}")
            xs = [I.rank_inputs("normal", "bf16", 8, size // 2, 3, si, k, 0.5) for k in range(2)]
            for algo in ("twoshot", "oneshot_sentinel"):
                _bench_sets(h, xs, algo, "bf16")


def test_full_size_c4_sixteen_ranks():
    """16 ranks, fp32 uniform[-1,1], 4 KiB .. 4 MiB: LL128-style atomic, one-shot LL, barrier
    baseline."""
    from latency_collectives_amd import inputs as I

    wl = I.WORKLOADS[4]
    with handle(16, max(wl["sizes"]), "f32") as h:
        for si, size in enumerate(wl["sizes"]):
            x = I.rank_inputs("uniform", "f32", 16, size // 4, 4, si, 0)
            for algo in ("ll128_atomic", "oneshot_ll", "barrier2"):
                _say(f"case c4 size={size} algo={algo}")
                got = run_allreduce(h, x, algo)
                assert_matches(got, x, algo, "f32")


def _device_check(outs, want: np.ndarray):
    """All ranks' outputs equal rank 0's (on the device); rank 0's equals `want` bit for bit."""
    import torch

    for r in range(1, len(outs)):
        assert torch.equal(outs[r], outs[0]), f"rank {r} output differs from rank 0"
    got = outs[0].cpu().numpy()
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, f"mismatch at {bad[:8]}: got {got[bad[:8]]} want {want[bad[:8]]}"


@pytest.mark.parametrize("size_mib", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["i32", "f32"])
def test_full_size_c5_twoshot(dtype, size_mib):
    """8 ranks, 16 .. 256 MiB per rank, two-shot in the benchmark's launch shape: int32
    uniform in [-2^20, 2^20] and fp32 uniform[-1,1], every element against the oracle."""
    from latency_collectives_amd import _ar as A
    from latency_collectives_amd import inputs as I
    from oracle import oracle
    import torch

    n = 8
    count = (size_mib << 20) // 4
    dist = "int20" if dtype == "i32" else "uniform"
    _say(f"case c5 dtype={dtype} size={size_mib} MiB")
    with handle(n, size_mib << 20, dtype) as h:
        ins = I.device_draw(dist, dtype, n, count, 5, size_mib, 0)
        outs = [torch.empty_like(t) for t in ins]
        A.ar_allreduce(h, ins, outs, count, A.AR_TWOSHOT)
        A.ar_check(h)
        host = [t.cpu().numpy() for t in ins]
        want = oracle.allreduce(host)[0]
        del host
        _device_check(outs, want)


def test_full_size_c5_rank_constant():
    """Rank r filled with r at 64 MiB per rank: every element of every output is N(N-1)/2."""
    from latency_collectives_amd import _ar as A
    from latency_collectives_amd import inputs as I
    import torch

    n, count = 8, (64 << 20) // 4
    with handle(n, 64 << 20, "i32") as h:
        ins = I.device_draw("rankconst", "i32", n, count, 5, 0, 0)
        outs = [torch.empty_like(t) for t in ins]
        A.ar_allreduce(h, ins, outs, count, A.AR_TWOSHOT)
        A.ar_check(h)
        for r in range(n):
            assert bool(torch.all(outs[r] == n * (n - 1) // 2)), f"rank {r}"


def test_alg_bytes_follow_the_launched_kernel():
    """ar_alg_bytes counts each logical read and write once for the protocol actually used: the
    one-pass two-shot re-arms sentinels (58 S at N = 8), the bulk two-shot uses completion flags
    and stores the all-gather straight into the outputs (30 S)."""
    from latency_collectives_amd import _ar as A

    n = 8
    with handle(n, 64 << 20, "f32") as h:
        s_small, s_big = 4096 * 4, 16 << 20
        assert A.ar_alg_bytes(h, s_small // 4, A.AR_TWOSHOT) == (n + 1) * s_small + 7 * (n - 1) * s_small
        assert A.ar_alg_bytes(h, s_big // 4, A.AR_TWOSHOT) == 2 * n * s_big + 2 * (n - 1) * s_big
        assert A.ar_alg_bytes(h, 1000, A.AR_ONESHOT_LL) == 2 * n * 4000 + 4 * n * (n - 1) * 4000
        assert A.ar_alg_bytes(h, 0, A.AR_ONESHOT_SENTINEL) == 0


def test_launch_shape_beyond_co_residency_is_refused():
    """Asking for more workgroups per rank than can be resident at once fails with AR_ENORES
    before anything is launched (a persistent grid that is not co-resident would never finish)."""
    from latency_collectives_amd import _ar as A
    import torch

    n, count = 16, 1 << 20
    with handle(n, count * 4, "f32", ctas=256) as h:
        x = [torch.zeros(count, device="cuda") for _ in range(n)]
        y = [torch.empty_like(t) for t in x]
        with pytest.raises(A.ArError) as e:
            A.ar_allreduce(h, x, y, count, A.AR_ONESHOT_SENTINEL)
        assert e.value.code == A.AR_ENORES
        # the handle stays usable with the automatic shape
        A.ar_set_option(h, A.AR_OPT_CTAS, 0)
        A.ar_allreduce(h, x, y, count, A.AR_ONESHOT_SENTINEL)
        A.ar_check(h)
        assert bool(torch.all(y[3] == 0))



@pytest.mark.parametrize("algo", ["twoshot", "oneshot_sentinel", "ll128_atomic", "oneshot_ll"])
def test_largest_message_a_handle_takes(algo):
    """The largest message per rank the boundary accepts (max_bytes < 2^31): 2 ranks, int32,
    2^31 - 64 bytes per rank, with inputs whose sums have a closed form (rank r element i =
    (i mod 4093) + 7919 r, so every output element is 2 (i mod 4093) + 7919), checked on the
    device for every element; one element more is refused (AR_ETOOBIG)."""
    import torch

    from latency_collectives_amd import _ar as A

    n = 2
    nbytes = (1 << 31) - 64
    count = nbytes // 4
    base = torch.arange(count, dtype=torch.int64, device="cuda") % 4093
    ins = [(base + 7919 * r).to(torch.int32) for r in range(n)]
    want = (2 * base + 7919).to(torch.int32)
    del base
    outs = [torch.empty_like(ins[0]) for _ in range(n)]
    print(f"case {algo} count={count}", flush=True)
    with handle(n, nbytes, "i32") as h:
        A.ar_allreduce(h, ins, outs, count, A.ALGOS[algo])
        A.ar_check(h)
        for r in range(n):
            assert torch.equal(outs[r], want), f"rank {r}"
        with pytest.raises(A.ArError) as e:
            A.ar_allreduce(h, ins, outs, count + 16, A.ALGOS[algo])
        assert e.value.code == A.AR_ETOOBIG
