"""GPU parity of the peer-split one-pass kernels (5..16 ranks: the waves of a workgroup share a
chunk's units and split the peers), through the C ABI, against the CPU oracle: bit-exact for
every dtype (the rank-order fold is unchanged), equal to the unsplit kernels, in persistent
loops with rank drift, and with a withheld rank (a bounded timeout, never a hang)."""

import numpy as np
import pytest

from tests.gpu_util import (assert_matches, draw, elem_bytes, from_device, handle, run_allreduce,
                            to_device)

pytestmark = pytest.mark.gpu

SPLIT_KERNELS = {26, 27, 28, 29, 33}
LL128_SPLIT = {30, 31, 32}
COUNTS = [1, 7, 33, 64, 1000, 4097]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [5, 6, 7, 8, 12, 16])
def test_split_matches_oracle_and_unsplit(n, dtype):
    from latency_collectives_amd import _ar as A

    algos = ["oneshot_sentinel", "oneshot_ll"] + (["twoshot"] if dtype != "i32" else [])
    for algo in algos:
        for count in COUNTS + [n * 517 + 3]:
            if dtype == "bf16" and count % 2 == 0:
                count += 1  # odd bf16 lengths: the 2-byte tail path
            x = draw(dtype, n, count, seed=1000 * n + count)
            with handle(n, count * elem_bytes(dtype), dtype) as h:
                plan = A.ar_plan_info(h, count, A.ALGOS[algo])
                _say(f"case n={n} {dtype} {algo} count={count} plan={plan}")
                got = run_allreduce(h, x, algo)
                assert_matches(got, x, algo, dtype)
                A.ar_set_option(h, A.AR_OPT_SPLIT, 0)
                plain = A.ar_plan_info(h, count, A.ALGOS[algo])
                assert plain["kernel"] not in SPLIT_KERNELS
                ref = run_allreduce(h, x, algo)
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))
            if count <= 1000:
                assert plan["kernel"] in SPLIT_KERNELS, plan
                assert plan["threads"] == 256


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [6, 8, 16])
def test_split_with_16_byte_units(n, dtype):
    """AR_OPT_NARROW = 0: the peer-split kernels with 16-byte units (families 26 and 28), equal
    to the oracle and to the 8-byte-unit split kernels."""
    from latency_collectives_amd import _ar as A

    for algo, fam in (("oneshot_sentinel", 26), ("twoshot", 28)):
        for count in (1, 9, 333, 64 * n + 7):
            if dtype == "bf16" and count % 2 == 0:
                count += 1
            x = draw(dtype, n, count, seed=7000 + n * count)
            with handle(n, count * elem_bytes(dtype), dtype, narrow=0) as h:
                plan = A.ar_plan_info(h, count, A.ALGOS[algo])
                _say(f"case n={n} {dtype} {algo} count={count} plan={plan}")
                assert plan["kernel"] == fam and plan["unit_bytes"] == 16, plan
                got = run_allreduce(h, x, algo)
                assert_matches(got, x, algo, dtype)
                A.ar_set_option(h, A.AR_OPT_NARROW, 1)
                ref = run_allreduce(h, x, algo)
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))


def test_split_kernels_planned_for_the_decode_shapes():
    """8 ranks, bf16 [tokens, 8192]: the kernels split while a chunk's 64-unit blocks get a
    compute unit each (32 per rank): the two-shot up to 8 tokens, the one-shot at 1 token (2048
    8-byte units); beyond that, and with 4 ranks, the unsplit kernels."""
    from latency_collectives_amd import _ar as A

    with handle(8, 64 * 8192 * 2, "bf16") as h:
        for tokens in (1, 2, 4, 8, 16):
            for algo in ("twoshot", "oneshot_sentinel"):
                p = A.ar_plan_info(h, tokens * 8192, A.ALGOS[algo])
                _say(f"tokens={tokens} {algo}: {p}")
                want = tokens <= 8 if algo == "twoshot" else tokens == 1
                assert (p["kernel"] in SPLIT_KERNELS) == want, p
                if want:
                    assert p["ctas"] <= 32
    with handle(4, 4096, "bf16") as h:
        assert A.ar_plan_info(h, 1024, A.AR_ONESHOT_SENTINEL)["kernel"] not in SPLIT_KERNELS


@pytest.mark.parametrize("algo", ["oneshot_sentinel", "oneshot_ll", "twoshot"])
@pytest.mark.parametrize("n", [8, 16])
def test_split_persistent_loop_with_drift(n, algo):
    """60 back-to-back AllReduces over 6 input sets with random per-rank delays, every set
    checked (the double-buffer credit and the LDS exchange buffers under rank skew)."""
    import torch

    from latency_collectives_amd import _ar as A

    count = 2048 + 5  # split at 8 and 16 ranks (a 64-unit block per compute unit)
    xs = [draw("bf16", n, count, seed=77 + k) for k in range(6)]
    with handle(n, count * 2, "bf16", drift=3) as h:
        assert A.ar_plan_info(h, count, A.ALGOS[algo])["kernel"] in SPLIT_KERNELS
        ins = [t for x1 in xs for t in to_device(x1)]
        outs = [torch.empty_like(t) for t in ins]
        A.ar_bench(h, ins, outs, len(xs), count, A.ALGOS[algo], 60)
        for k, x1 in enumerate(xs):
            assert_matches(from_device(outs[k * n:(k + 1) * n], x1.dtype), x1, algo, "bf16")


@pytest.mark.parametrize("algo", ["oneshot_sentinel", "oneshot_ll", "twoshot"])
def test_split_withheld_rank_times_out(algo):
    """A rank that sends nothing: its peers' polls time out (bounded), every wave of a split
    workgroup leaves the step, and the handle reports AR_ETIMEOUT."""
    from latency_collectives_amd import _ar as A

    n, count = 8, 4096
    x = draw("f32", n, count, seed=5)
    with handle(n, count * 4, "f32", timeout_us=20000, withhold_rank=3) as h:
        assert A.ar_plan_info(h, count, A.ALGOS[algo])["kernel"] in SPLIT_KERNELS
        ins = to_device(x)
        import torch

        outs = [torch.empty_like(t) for t in ins]
        A.ar_allreduce(h, ins, outs, count, A.ALGOS[algo])
        torch.cuda.synchronize()
        with pytest.raises(A.ArError) as e:
            A.ar_check(h)
        assert e.value.code == A.AR_ETIMEOUT


def test_split_leaves_slots_rearmed():
    """After split calls of both algorithms every sentinel slot is armed again."""
    from latency_collectives_amd import _ar as A

    n = 8
    with handle(n, 8192 * 4, "f32") as h:
        for count in (100, 8192, 3):
            for algo in ("oneshot_sentinel", "twoshot"):
                x = draw("f32", n, count, seed=count)
                assert_matches(run_allreduce(h, x, algo), x, algo, "f32")
        for r in range(n):
            for reg in (A.REGION_P1, A.REGION_P2, A.REGION_P1_NEAR, A.REGION_P2_NEAR):
                w = A.ar_read_region(h, r, reg).view(np.uint32)
                assert np.all(w == 0xFFFFFFFF), f"rank {r} region {reg} not re-armed"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [5, 8, 12, 16])
def test_ll128_split_within_bound_and_dyadic_exact(n, dtype):
    """The peer-split LL128-style kernel: within the atomic-order bound on ragged counts (1, 2
    and 4 word slices per lane; blocks of 1 to 64 units, one or several per chunk), bit-exact on
    inputs whose partial sums are exact in any order, and its destinations and counters clear
    afterwards."""
    import torch

    from latency_collectives_amd import _ar as A

    eb = elem_bytes(dtype)
    counts = [1, 7, 33, 64 * n // eb + 5, 256 * n // eb + 3, 2048 * n // eb]
    with handle(n, (max(counts) + 1) * eb, dtype) as h:
        for count in counts:
            if dtype == "bf16" and count % 2 == 0:
                count += 1
            plan = A.ar_plan_info(h, count, A.AR_LL128_ATOMIC)
            _say(f"case n={n} {dtype} count={count} plan={plan}")
            assert plan["kernel"] in LL128_SPLIT, plan
            x = draw(dtype, n, count, seed=3000 + n + count)
            assert_matches(run_allreduce(h, x, "ll128_atomic"), x, "ll128_atomic", dtype)
            # dyadic values k * 2^-3, |k| <= 8: every partial sum is exact in fp32 and bf16
            g = np.random.default_rng(count)
            k = g.integers(-8, 8, size=(n, count), endpoint=True)
            xf = (k / 8.0).astype(np.float32)
            xd = (torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                  if dtype == "bf16" else xf)
            assert_matches(run_allreduce(h, xd, "ll128_atomic"), xd, "twoshot", dtype)
        for r in range(n):
            for reg in (A.REGION_ACC, A.REGION_CNT):
                w = A.ar_read_region(h, r, reg).view(np.uint32)
                assert np.all(w == 0), f"rank {r} region {reg} not clear"


def test_ll128_split_persistent_loop_and_timeout():
    """A persistent loop of 60 calls over 6 input sets with rank drift (every set within the
    bound), then a withheld rank ending in AR_ETIMEOUT."""
    import torch

    from latency_collectives_amd import _ar as A

    n, count = 16, 4096
    xs = [draw("f32", n, count, seed=500 + k) for k in range(6)]
    with handle(n, count * 4, "f32", drift=3) as h:
        assert A.ar_plan_info(h, count, A.AR_LL128_ATOMIC)["kernel"] in LL128_SPLIT
        ins = [t for x1 in xs for t in to_device(x1)]
        outs = [torch.empty_like(t) for t in ins]
        A.ar_bench(h, ins, outs, len(xs), count, A.AR_LL128_ATOMIC, 60)
        for k, x1 in enumerate(xs):
            assert_matches(from_device(outs[k * n:(k + 1) * n], x1.dtype), x1, "ll128_atomic",
                           "f32")
    x = xs[0]
    with handle(n, count * 4, "f32", timeout_us=20000, withhold_rank=5) as h:
        ins = to_device(x)
        outs = [torch.empty_like(t) for t in ins]
        A.ar_allreduce(h, ins, outs, count, A.AR_LL128_ATOMIC)
        torch.cuda.synchronize()
        with pytest.raises(A.ArError) as e:
            A.ar_check(h)
        assert e.value.code == A.AR_ETIMEOUT
