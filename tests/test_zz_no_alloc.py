"""The allocation-free AllReduce (ar_allreduce_noalloc) against ar_allreduce on a handle.

Both entry points run the same kernels; the allocation-free one keeps its scratch in a static
device array. Every case makes two calls in a row, the second with a smaller input, and
compares each output with the handle's output for the same inputs: bit for bit for the
fixed-order algorithms and int32, within the atomic-order bound N * 2^-23 * sum_r |x_r| for the
LL128-style fp32 path (whose order of additions may differ between any two runs).
"""

import numpy as np
import pytest

from tests.gpu_util import assert_matches, draw, elem_bytes, from_device, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run(A, n, dtype, x, algo, h=None):
    import torch

    ins = to_device(x)
    outs = [torch.full_like(t, 0x55) for t in ins]
    if h is None:
        A.ar_allreduce_noalloc(n, A.DTYPES[dtype], ins, outs, x.shape[1], A.ALGOS[algo])
    else:
        A.ar_allreduce(h, ins, outs, x.shape[1], A.ALGOS[algo])
    torch.cuda.synchronize()
    return from_device(outs, x.dtype)


def _same(got, ref, x, algo, dtype):
    n = x.shape[0]
    if algo == "ll128_atomic" and dtype == "f32":
        bound = n * 2.0 ** -23 * np.sum(np.abs(x.astype(np.float64)), axis=0)
        for r in range(n):
            err = np.abs(got[r].astype(np.float64) - ref[r].astype(np.float64))
            assert np.all(err <= 2 * bound), f"rank {r} beyond the atomic-order bound"
    else:
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), "outputs differ"


CASES = [
    # (nranks, dtype, algo, first count, second count)
    (2, "f32", "oneshot_ll", 32, 8),
    (4, "bf16", "oneshot_sentinel", 131072, 513),
    (8, "bf16", "twoshot", 65536, 8192),
    (16, "f32", "ll128_atomic", 65536, 1000),
    (8, "i32", "twoshot", 1 << 20, 4097),
    (16, "f32", "oneshot_sentinel", 70001, 33),
    (3, "i32", "auto", 100003, 7),
    (16, "bf16", "barrier2", 40000, 17),
    (8, "f32", "twoshot", 1 << 22, 1 << 12),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}" for c in CASES])
def test_noalloc_matches_handle(case):
    from latency_collectives_amd import _ar as A
    from tests.gpu_util import handle

    n, dtype, algo, c1, c2 = case
    with handle(n, c1 * elem_bytes(dtype), dtype) as h:
        for k, count in enumerate((c1, c2)):
            _say(f"case n={n} dtype={dtype} algo={algo} count={count}")
            x = draw(dtype, n, count, seed=700 + 10 * n + k)
            ref = _run(A, n, dtype, x, algo, h)
            got = _run(A, n, dtype, x, algo)
            _same(got, ref, x, algo, dtype)
            assert_matches(got, x, algo, dtype)


def test_noalloc_repeated_layouts_and_errors():
    """Switching rank count and dtype between calls re-lays the array out; repeated calls with one
    layout keep going from the stored sequence number; bad arguments are refused."""
    from latency_collectives_amd import _ar as A
    import torch

    for n, dtype in ((4, "f32"), (4, "f32"), (2, "bf16"), (16, "i32"), (4, "f32")):
        for count in (1000, 17):
            _say(f"case n={n} dtype={dtype} count={count}")
            x = draw(dtype, n, count, seed=n + count)
            got = _run(A, n, dtype, x, "oneshot_sentinel")
            assert_matches(got, x, "oneshot_sentinel", dtype)
    t = [torch.zeros(4, device="cuda") for _ in range(2)]
    with pytest.raises(A.ArError) as e:
        A.ar_allreduce_noalloc(17, A.AR_FLOAT32, t + t * 8, t + t * 8, 4, A.AR_ONESHOT_LL)
    assert e.value.code == A.AR_EINVAL
    with pytest.raises(A.ArError) as e:
        A.ar_allreduce_noalloc(2, A.AR_FLOAT32, t, t, 1 << 30, A.AR_ONESHOT_LL)
    assert e.value.code == A.AR_ETOOBIG
    with pytest.raises(A.ArError) as e:
        A.ar_allreduce_noalloc(2, 9, t, t, 4, A.AR_ONESHOT_LL)
    assert e.value.code == A.AR_EINVAL
