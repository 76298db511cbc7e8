"""GPU parity of the LL128-style atomic AllReduce beyond fp32: the bf16 path (packed bf16 atomic
additions, rounding at every addition) and the deterministic variant (groups of ranks added in a
fixed order), through the C ABI, against the CPU oracle.

Bars: the deterministic variant equals the oracle's grouped fold (groups of AR_OPT_GROUP
consecutive ranks in rank order, then the group sums in group order) bit for bit, on every run
and in every launch shape; the bf16 atomic path is within N * 2^-8 * sum_r |x_r| per element of
the rank-order oracle (plus N subnormal spacings) and bit-exact on inputs whose partial sums are
all exact in bf16.
"""

import numpy as np
import pytest

from tests.gpu_util import (assert_matches, draw, elem_bytes, from_device, handle, run_allreduce,
                            to_device)

pytestmark = pytest.mark.gpu

COUNTS = [1, 7, 33, 1000, 4099, 70001]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 8, 16])
def test_deterministic_matches_grouped_oracle(n, dtype):
    for group in (2, 3, 4, 16):
        with handle(n, max(COUNTS) * elem_bytes(dtype), dtype, group=group) as h:
            for i, count in enumerate(COUNTS):
                _say(f"case n={n} dtype={dtype} group={group} count={count}")
                x = draw(dtype, n, count, seed=400 * n + 10 * group + i)
                got = run_allreduce(h, x, "ll128_det")
                assert_matches(got, x, "ll128_det", dtype, group=group)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic_is_bit_reproducible(dtype):
    """The same inputs give the same bits on every run, whatever the launch shape (one 64-thread
    workgroup per rank, or the planner's), and in a persistent loop of back-to-back calls with
    random per-rank delays."""
    from latency_collectives_amd import _ar as A

    n, count = 16, 70001
    x = draw(dtype, n, count, seed=77)
    runs = []
    for ctas, threads in ((0, 0), (1, 64), (3, 128)):
        with handle(n, count * elem_bytes(dtype), dtype, ctas=ctas, threads=threads) as h:
            for rep in range(4):
                _say(f"case dtype={dtype} ctas={ctas} threads={threads} rep={rep}")
                runs.append(run_allreduce(h, x, "ll128_det"))
    for got in runs[1:]:
        assert np.array_equal(got.view(np.uint8), runs[0].view(np.uint8))
    assert_matches(runs[0], x, "ll128_det", dtype)
    # persistent loop: 30 calls over 6 input sets with rank drift, every set checked
    import torch

    xs = [draw(dtype, n, 4096, seed=900 + k) for k in range(6)]
    with handle(n, 4096 * elem_bytes(dtype), dtype, drift=3) as h:
        ins = [t for x1 in xs for t in to_device(x1)]
        outs = [torch.empty_like(t) for t in ins]
        A.ar_bench(h, ins, outs, len(xs), 4096, A.AR_LL128_DET, 30)
        for k, x1 in enumerate(xs):
            got = from_device(outs[k * n:(k + 1) * n], x1.dtype)
            assert_matches(got, x1, "ll128_det", dtype)


def test_deterministic_int32_is_the_exact_sum():
    """int32: the deterministic entry point runs the plain atomic kernel (integer addition does
    not depend on the order); results equal the oracle, sums equal to INT32_MIN included."""
    for n in (3, 16):
        x = draw("i32", n, 10001, seed=n)
        with handle(n, 10001 * 4, "i32") as h:
            got = run_allreduce(h, x, "ll128_det")
        assert_matches(got, x, "twoshot", "i32")


def test_deterministic_leaves_scratch_clear():
    """After deterministic and plain atomic calls alternate on one handle, every destination and
    every ticket and counter is back to zero (the next call of either kind starts clean)."""
    from latency_collectives_amd import _ar as A

    n = 8
    for dtype in ("f32", "bf16"):
        with handle(n, 20000 * 4, dtype) as h:
            for it in range(3):
                for algo, count in (("ll128_det", 20000), ("ll128_atomic", 999),
                                    ("ll128_det", 77), ("ll128_atomic", 20000)):
                    x = draw(dtype, n, count, seed=it * 10 + count % 13)
                    got = run_allreduce(h, x, algo)
                    assert_matches(got, x, algo, dtype)
            for r in range(n):
                for reg in (A.REGION_ACC, A.REGION_CNT, A.REGION_SINK):
                    w = A.ar_read_region(h, r, reg).view(np.uint32)
                    assert np.all(w == 0), f"{dtype} rank {r} region {reg} not clear"


@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_bf16_atomic_within_bound(n):
    for i, count in enumerate(COUNTS):
        _say(f"case n={n} count={count}")
        x = draw("bf16", n, count, seed=600 + 10 * n + i)
        with handle(n, count * 2, "bf16") as h:
            got = run_allreduce(h, x, "ll128_atomic")
        assert_matches(got, x, "ll128_atomic", "bf16")


def test_bf16_atomic_exact_on_dyadic_inputs():
    """bf16 inputs k * 2^-3 with |k| <= 8: every partial sum of up to 16 of them is a multiple of
    2^-3 below 16 in magnitude, exact in bf16's 8 significant bits, so any order of atomic
    additions gives the oracle's result bit for bit."""
    import torch

    for n in (2, 5, 16):
        g = np.random.default_rng(n)
        k = g.integers(-8, 8, size=(n, 5003), endpoint=True)
        xb = torch.from_numpy((k / 8.0).astype(np.float32)).to(torch.bfloat16)
        x = xb.view(torch.int16).numpy().view(np.uint16).copy()
        with handle(n, x.shape[1] * 2, "bf16") as h:
            got = run_allreduce(h, x, "ll128_atomic")
        assert_matches(got, x, "twoshot", "bf16")  # bit-exact bar


def test_bf16_atomic_rounding_probe():
    """Two ranks, 1 + 2^-7 and 2^-8: the sum 1 + 3 * 2^-8 is a tie between 1 + 2^-7 (odd) and
    1 + 2^-6 (even). The oracle rounds it to even; a packed bf16 atomic that rounds to nearest
    even gives the same, one that truncates gives 1 + 2^-7. Either is within the bound; the
    test records which the hardware does."""
    x = np.array([[0x3F81] * 64, [0x3B80] * 64], dtype=np.uint16)
    with handle(2, 128, "bf16") as h:
        got = run_allreduce(h, x, "ll128_atomic")
    _say(f"packed bf16 atomic: 0x3F81 + 0x3B80 -> {got[0][0]:#06x} (nearest even: 0x3f82)")
    assert set(got[0].tolist()) <= {0x3F82, 0x3F81}
    assert_matches(got, x, "ll128_atomic", "bf16")
