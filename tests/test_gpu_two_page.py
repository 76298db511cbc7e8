"""GPU parity of the one-pass two-shot and one-shot LL on two-page near slots (more than 8 ranks,
messages whose 2 N slots need more than one near page: buffer b of the p1 and p2 (two-shot) or
ll (LL) near regions in page b, the
second buffer at its page's start or one granule before it), through the C ABI, against the CPU
oracle: bit-exact for fp32 and bf16, equal to the same call on regular slots, in persistent loops
with rank drift, the slots re-armed afterwards, and a withheld rank ending in a bounded timeout."""

import contextlib

import numpy as np
import pytest

from tests.gpu_util import (assert_matches, draw, elem_bytes, from_device, handle, run_allreduce,
                            to_device)

pytestmark = pytest.mark.gpu

# bytes per rank at 16 ranks: just above the one-page limit (32 KiB partitions, ragged), between,
# and the largest whose 16 slots of one buffer fill one page (64 KiB partitions)
SIZES16 = [524288 + 16, 786432 + 48, 1048576]


def _say(*a):
    print(*a, flush=True)


@contextlib.contextmanager
def two_page_handle(n, max_bytes, dtype, count, **opts):
    """A handle whose plan for `count` uses two-page slots (whatever the calibration of the second
    pages said: mirrored pages move buffer 1 one granule down, others keep it at the page)."""
    from latency_collectives_amd import _ar as A

    with handle(n, max_bytes, dtype, **opts) as h:
        plan = A.ar_plan_info(h, count, A.AR_TWOSHOT)
        assert plan["near"] == 3, plan
        yield h


def _sentinel(dtype):
    return {"f32": 0xFFFFFFFF, "bf16": 0xFFFFFFFF, "i32": 0x80000000}[dtype]


@pytest.mark.parametrize("n,dtype,sizes", [(16, "f32", SIZES16), (16, "bf16", SIZES16),
                                           (12, "f32", [786432 + 4])])
def test_two_page_matches_oracle_and_regular_slots(n, dtype, sizes):
    from latency_collectives_amd import _ar as A

    eb = elem_bytes(dtype)
    with two_page_handle(n, max(sizes), dtype, max(sizes) // eb) as h:
        for size in sizes:
            count = size // eb
            if dtype == "bf16" and count % 2 == 0:
                count -= 1  # odd bf16 lengths: the 2-byte tail path
            plan = A.ar_plan_info(h, count, A.AR_TWOSHOT)
            _say(f"case n={n} {dtype} count={count} plan={plan}")
            assert plan["near"] == 3, plan
            assert plan["kernel"] == 34, plan
            x = draw(dtype, n, count, seed=5000 + count)
            got = run_allreduce(h, x, "twoshot")
            assert_matches(got, x, "twoshot", dtype)
            got2 = run_allreduce(h, x, "twoshot")  # the other buffer (page)
            assert np.array_equal(got.view(np.uint8), got2.view(np.uint8))
            A.ar_set_option(h, A.AR_OPT_TWO_PAGE, 0)
            regular = A.ar_plan_info(h, count, A.AR_TWOSHOT)
            assert regular["near"] == 0, regular
            ref = run_allreduce(h, x, "twoshot")
            A.ar_set_option(h, A.AR_OPT_TWO_PAGE, 1)
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))
        for r in range(n):
            for region in (A.REGION_P1_NEAR, A.REGION_P2_NEAR):
                w = A.ar_read_region(h, r, region).view(np.uint32)
                assert w.size * 4 == 2 * (2 << 20), w.size
                assert np.all(w == _sentinel(dtype)), f"rank {r} region {region}: not re-armed"


def test_two_page_only_where_planned():
    """Small messages of a two-page handle stay on the one-page near slots; the int32 two-shot
    (the bulk kernel), the 8-rank two-shot (the bulk kernel is faster there) and other placements
    never take two-page slots; the option takes 0 and 1 only."""
    from latency_collectives_amd import _ar as A

    with handle(16, 1 << 20, "f32") as h:
        assert A.ar_plan_info(h, 4096, A.AR_TWOSHOT)["near"] == 1
        assert A.ar_plan_info(h, 1 << 18, A.AR_ONESHOT_SENTINEL)["near"] != 3
        A.ar_set_option(h, A.AR_OPT_PLACEMENT, A.AR_PLACE_SAME)
        assert A.ar_plan_info(h, 1 << 18, A.AR_TWOSHOT)["near"] != 3
        with pytest.raises(A.ArError) as e:
            A.ar_set_option(h, A.AR_OPT_TWO_PAGE, 2)
        assert e.value.code == A.AR_EINVAL
    with handle(16, 1 << 20, "i32") as h:
        assert A.ar_plan_info(h, 1 << 18, A.AR_TWOSHOT)["near"] == 0
    with handle(8, 1 << 20, "f32") as h:
        assert A.ar_plan_info(h, 1 << 18, A.AR_TWOSHOT)["near"] != 3
        # p2 keeps one page at 8 ranks; p1 has two for the one-shot sentinel's slots
        assert A.ar_region_bytes(h, A.REGION_P2_NEAR) == 2 << 20
        assert A.ar_region_bytes(h, A.REGION_P1_NEAR) == 4 << 20


def test_two_page_persistent_loop_with_drift():
    """60 back-to-back AllReduces over 3 input sets with random per-rank delays, both buffers
    (pages) in turn, every set checked."""
    import torch

    from latency_collectives_amd import _ar as A

    n, count = 16, (1 << 20) // 4
    xs = [draw("f32", n, count, seed=950 + k) for k in range(3)]
    with two_page_handle(n, 1 << 20, "f32", count, drift=3) as h:
        ins = [t for x1 in xs for t in to_device(x1)]
        outs = [torch.empty_like(t) for t in ins]
        A.ar_bench(h, ins, outs, len(xs), count, A.AR_TWOSHOT, 60)
        for k, x1 in enumerate(xs):
            assert_matches(from_device(outs[k * n:(k + 1) * n], x1.dtype), x1, "twoshot", "f32")


def test_two_page_withheld_rank_times_out():
    from latency_collectives_amd import _ar as A

    n, count = 16, (1 << 20) // 4
    x = draw("f32", n, count, seed=12)
    with two_page_handle(n, 1 << 20, "f32", count, timeout_us=20000, withhold_rank=5) as h:
        import torch

        ins = to_device(x)
        outs = [torch.empty_like(t) for t in ins]
        A.ar_allreduce(h, ins, outs, count, A.AR_TWOSHOT)
        torch.cuda.synchronize()
        with pytest.raises(A.ArError) as e:
            A.ar_check(h)
        assert e.value.code == A.AR_ETIMEOUT


# one-shot LL at 16 ranks: 16-byte lines of 8 bytes of payload, so the ll slots of a message
# above 16 KiB need two pages; 32 KiB fills one page with the 16 slots of one buffer
LL_SIZES16 = [16384 + 8, 24576 + 4, 32768]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
def test_two_page_oneshot_ll_matches_oracle_and_regular_slots(dtype):
    from latency_collectives_amd import _ar as A

    n, eb = 16, elem_bytes(dtype)
    with handle(n, max(LL_SIZES16), dtype) as h:
        for size in LL_SIZES16:
            count = size // eb
            if dtype == "bf16" and count % 2 == 0:
                count -= 1
            plan = A.ar_plan_info(h, count, A.AR_ONESHOT_LL)
            _say(f"case LL n={n} {dtype} count={count} plan={plan}")
            assert plan["near"] == 3 and plan["kernel"] == 35 and plan["unit_bytes"] == 8, plan
            x = draw(dtype, n, count, seed=5100 + count)
            got = run_allreduce(h, x, "oneshot_ll")
            assert_matches(got, x, "oneshot_ll", dtype)
            got2 = run_allreduce(h, x, "oneshot_ll")  # the other buffer (page)
            assert np.array_equal(got.view(np.uint8), got2.view(np.uint8))
            A.ar_set_option(h, A.AR_OPT_TWO_PAGE, 0)
            assert A.ar_plan_info(h, count, A.AR_ONESHOT_LL)["near"] == 0
            ref = run_allreduce(h, x, "oneshot_ll")
            A.ar_set_option(h, A.AR_OPT_TWO_PAGE, 1)
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))
        # a message that fits one page keeps the one-page slots
        assert A.ar_plan_info(h, 16384 // eb, A.AR_ONESHOT_LL)["near"] == 1


def test_two_page_oneshot_ll_persistent_loop_with_drift():
    import torch

    from latency_collectives_amd import _ar as A

    n, count = 16, 32768 // 4
    xs = [draw("f32", n, count, seed=960 + k) for k in range(3)]
    with handle(n, 32768, "f32", drift=3) as h:
        assert A.ar_plan_info(h, count, A.AR_ONESHOT_LL)["near"] == 3
        ins = [t for x1 in xs for t in to_device(x1)]
        outs = [torch.empty_like(t) for t in ins]
        A.ar_bench(h, ins, outs, len(xs), count, A.AR_ONESHOT_LL, 60)
        for k, x1 in enumerate(xs):
            assert_matches(from_device(outs[k * n:(k + 1) * n], x1.dtype), x1, "oneshot_ll", "f32")


# one-shot sentinel from 8 ranks on: its p1 slots hold a whole message, so above 64 KiB (8 ranks)
# or 32 KiB (16 ranks) they need two pages; 128 KiB and 64 KiB fill one page per buffer
SENT_CASES = [(8, [65536 + 16, 98304 + 4, 131072]), (16, [32768 + 16, 65536])]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n,sizes", SENT_CASES)
def test_two_page_oneshot_sentinel_matches_oracle_and_regular_slots(n, sizes, dtype):
    from latency_collectives_amd import _ar as A

    eb = elem_bytes(dtype)
    with handle(n, max(sizes), dtype) as h:
        for size in sizes:
            count = size // eb
            if dtype == "bf16" and count % 2 == 0:
                count -= 1
            plan = A.ar_plan_info(h, count, A.AR_ONESHOT_SENTINEL)
            _say(f"case sentinel n={n} {dtype} count={count} plan={plan}")
            assert plan["near"] == 3 and plan["kernel"] == 36, plan
            x = draw(dtype, n, count, seed=5200 + count)
            got = run_allreduce(h, x, "oneshot_sentinel")
            assert_matches(got, x, "oneshot_sentinel", dtype)
            got2 = run_allreduce(h, x, "oneshot_sentinel")  # the other buffer (page)
            assert np.array_equal(got.view(np.uint8), got2.view(np.uint8))
            A.ar_set_option(h, A.AR_OPT_TWO_PAGE, 0)
            assert A.ar_plan_info(h, count, A.AR_ONESHOT_SENTINEL)["near"] == 0
            ref = run_allreduce(h, x, "oneshot_sentinel")
            A.ar_set_option(h, A.AR_OPT_TWO_PAGE, 1)
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))
        for r in range(n):
            w = A.ar_read_region(h, r, A.REGION_P1_NEAR).view(np.uint32)
            assert w.size * 4 == 2 * (2 << 20), w.size
            assert np.all(w == _sentinel(dtype)), f"rank {r}: p1 near region not re-armed"
        if n == 8:  # the two-shot of 8 ranks keeps the bulk kernel on regular slots
            assert A.ar_plan_info(h, count, A.AR_TWOSHOT)["near"] != 3
