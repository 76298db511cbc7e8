"""GPU parity of the LL128-style kernel's all-gather with completion flags (the owners store their
sums straight into every rank's output, or into the peers' bulk all-gather slots when a
persistent launch's output sets overlap its input sets), through the C ABI, against the CPU
oracle: fp32 and bf16 within their bounds, int32 bit-exact, in place, persistent loops with
rank drift on distinct sets, and a persistent in-place loop that must take the slots."""

import numpy as np
import pytest

from tests.gpu_util import (assert_matches, draw, from_device, handle, run_allreduce, to_device)

pytestmark = pytest.mark.gpu

# (ranks, bytes per rank): one wave, one pass over several workgroups, several passes, chunked
CASES = [(2, 4096 + 12), (5, 65536 + 20), (8, 262144), (16, 1048576 + 48)]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n,size", CASES)
def test_ll128_flag_allgather_matches_oracle(n, size, dtype):
    """The plain kernel (peer-split off) at every shape, out of place and in place."""
    from latency_collectives_amd import _ar as A

    eb = 2 if dtype == "bf16" else 4
    count = size // eb
    if dtype == "bf16" and count % 2 == 0:
        count -= 1  # odd bf16 lengths: the 2-byte tail path
    x = draw(dtype, n, count, seed=6000 + n * 7 + count % 97)
    with handle(n, size, dtype, split=0) as h:
        plan = A.ar_plan_info(h, count, A.AR_LL128_ATOMIC)
        _say(f"case n={n} {dtype} count={count} plan={plan}")
        assert plan["kernel"] in (4, 22, 23), plan
        got = run_allreduce(h, x, "ll128_atomic")
        assert_matches(got, x, "ll128_atomic", dtype)
        got_in = run_allreduce(h, x, "ll128_atomic", inplace=True)
        assert_matches(got_in, x, "ll128_atomic", dtype)
        if dtype == "i32":
            assert np.array_equal(got, got_in)


@pytest.mark.parametrize("dtype", ["f32", "i32"])
def test_ll128_flag_allgather_persistent_loop_with_drift(dtype):
    """40 back-to-back AllReduces over 4 distinct input sets (outputs stored by the owners) with
    random per-rank delays, every set checked."""
    import torch

    from latency_collectives_amd import _ar as A

    n, count = 16, 65536
    xs = [draw(dtype, n, count, seed=620 + k) for k in range(4)]
    with handle(n, count * 4, dtype, split=0, drift=3) as h:
        ins = [t for x1 in xs for t in to_device(x1)]
        outs = [torch.empty_like(t) for t in ins]
        A.ar_bench(h, ins, outs, len(xs), count, A.AR_LL128_ATOMIC, 40)
        for k, x1 in enumerate(xs):
            assert_matches(from_device(outs[k * n:(k + 1) * n], x1.dtype), x1, "ll128_atomic",
                           dtype)


def test_ll128_persistent_in_place_loop_takes_the_slots():
    """A persistent in-place loop on one set (each iteration reduces the previous result): the
    outputs overlap the inputs, so the owners put the all-gather into the peers' slots; after k
    iterations every element is N^(k-1) times the first sum (wrapping int32)."""
    from latency_collectives_amd import _ar as A

    n, count, iters = 8, 70001, 3
    x = draw("i32", n, count, seed=79)
    with handle(n, count * 4, "i32") as h:
        bufs = to_device(x)
        A.ar_bench(h, bufs, bufs, 1, count, A.AR_LL128_ATOMIC, iters)
        got = from_device(bufs, np.int32)
    first = x.astype(np.int64).sum(axis=0)
    want = ((first * n ** (iters - 1) + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int32)
    for r in range(n):
        assert np.array_equal(got[r], want), f"rank {r}"


def test_ll128_flag_allgather_withheld_rank_times_out():
    from latency_collectives_amd import _ar as A

    n, count = 8, 65536
    x = draw("f32", n, count, seed=13)
    with handle(n, count * 4, "f32", split=0, timeout_us=20000, withhold_rank=3) as h:
        import torch

        ins = to_device(x)
        outs = [torch.empty_like(t) for t in ins]
        A.ar_allreduce(h, ins, outs, count, A.AR_LL128_ATOMIC)
        torch.cuda.synchronize()
        with pytest.raises(A.ArError) as e:
            A.ar_check(h)
        assert e.value.code == A.AR_ETIMEOUT
