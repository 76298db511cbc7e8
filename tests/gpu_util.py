"""Helpers for the GPU tests: move seeded inputs to the device, run the C ABI, compare with the
oracle at the tolerances the method allows."""

from __future__ import annotations

import contextlib
import math
import os

import numpy as np

from latency_collectives_amd import inputs as I

ALGO_NAMES = ["oneshot_ll", "oneshot_sentinel", "twoshot", "ll128_atomic", "barrier2",
              "ll128_det"]
FIXED_ORDER = {"oneshot_ll", "oneshot_sentinel", "twoshot", "barrier2"}
DET_GROUP = 2  # the deterministic LL128-style variant's default ranks per group


def torch_mod():
    import torch

    return torch


def to_device(x: np.ndarray) -> list:
    """[N, count] host array -> N separate device tensors holding the same bytes."""
    torch = torch_mod()
    out = []
    for r in range(x.shape[0]):
        row = np.ascontiguousarray(x[r])
        if row.dtype == np.uint16:
            row = row.view(np.int16)
        out.append(torch.from_numpy(row.copy()).cuda())
    return out


def from_device(ts: list, np_dtype) -> np.ndarray:
    rows = [t.cpu().numpy() for t in ts]
    return np.stack([r.view(np_dtype) for r in rows])


@contextlib.contextmanager
def handle(nranks: int, max_bytes: int, dtype: str, env: dict | None = None, **opts):
    from latency_collectives_amd import _ar as A

    saved = {}
    for k, v in (env or {}).items():
        saved[k] = os.environ.get(k)
        os.environ[k] = str(v)
    try:
        h = A.ar_create(nranks, max_bytes, A.DTYPES[dtype])
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    try:
        for k, v in opts.items():
            A.ar_set_option(h, getattr(A, "AR_OPT_" + k.upper()), v)
        yield h
    finally:
        A.ar_destroy(h)


def run_allreduce(h, x: np.ndarray, algo: str, inplace: bool = False) -> np.ndarray:
    from latency_collectives_amd import _ar as A

    ins = to_device(x)
    torch = torch_mod()
    outs = ins if inplace else [torch.full_like(t, 0x55) for t in ins]
    A.ar_allreduce(h, ins, outs, x.shape[1], A.ALGOS[algo])
    A.ar_check(h)
    return from_device(outs, x.dtype)


def oracle_sum(x: np.ndarray) -> np.ndarray:
    from oracle import oracle

    return oracle.allreduce([np.ascontiguousarray(x[r]) for r in range(x.shape[0])])[0]


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |v| (binary32 values v); subnormal spacing below 2^-126."""
    a = np.abs(v.astype(np.float64))
    out = np.full(a.shape, 2.0 ** -133)
    nz = a >= 2.0 ** -126
    out[nz] = 2.0 ** (np.floor(np.log2(a[nz])) - 7)
    return out


def widen_bf16(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def assert_matches(got: np.ndarray, x: np.ndarray, algo: str, dtype: str,
                   group: int = DET_GROUP) -> None:
    """got: [N, count] GPU outputs; x: [N, count] inputs. The deterministic LL128-style variant is
    compared with the oracle's grouped fold (groups of `group` ranks), bit for bit."""
    if algo == "ll128_det" and dtype != "i32":
        from oracle import oracle

        want = oracle.allreduce_grouped([np.ascontiguousarray(x[r]) for r in range(x.shape[0])],
                                        group)[0]
        for r in range(x.shape[0]):
            bad = np.nonzero(got[r].view(np.uint8) != want.view(np.uint8))[0]
            assert bad.size == 0, f"rank {r}: deterministic variant differs at byte {bad[:8]}"
        return
    want = oracle_sum(x)
    n = x.shape[0]
    for r in range(n):
        assert np.array_equal(got[r].view(np.uint8), got[0].view(np.uint8)), \
            f"rank {r} output differs from rank 0"
    g = got[0]
    if dtype == "i32":
        bad = np.nonzero(g != want)[0]
        assert bad.size == 0, f"int32 mismatch at {bad[:8]}: got {g[bad[:8]]} want {want[bad[:8]]}"
        return
    if algo in FIXED_ORDER:
        # Fixed rank order: the GPU fold is the oracle's fold, bit for bit.
        bad = np.nonzero(g.view(np.uint32 if dtype == "f32" else np.uint16)
                         != want.view(np.uint32 if dtype == "f32" else np.uint16))[0]
        if dtype == "bf16" and bad.size:
            # the stated bound is one bf16 ulp of the oracle's result; report both
            diff = np.abs(widen_bf16(g[bad]).astype(np.float64)
                          - widen_bf16(want[bad]).astype(np.float64))
            within = bool(np.all(diff <= bf16_ulp(widen_bf16(want[bad]))))
            raise AssertionError(f"bf16 not bit-exact at {bad[:8]} (within 1 ulp: {within})")
        assert bad.size == 0, f"fp32 mismatch at {bad[:8]}: got {g[bad[:8]]} want {want[bad[:8]]}"
        return
    if dtype == "bf16":
        # Atomic order with bf16 accumulation (packed bf16 atomics round at every addition):
        # |gpu - oracle| <= N * 2^-8 * sum_r |x_r| per element, plus N subnormal spacings.
        xs = widen_bf16(x).astype(np.float64)
        bound = n * 2.0 ** -8 * np.sum(np.abs(xs), axis=0) + n * 2.0 ** -133
        err = np.abs(widen_bf16(g).astype(np.float64) - widen_bf16(want).astype(np.float64))
        bad = np.nonzero(err > bound)[0]
        assert bad.size == 0, f"atomic-order bf16 beyond bound at {bad[:8]}: err {err[bad[:8]]}"
        return
    # Atomic order (LL128-style): |gpu - oracle| <= N * 2^-23 * sum_r |x_r| per element.
    bound = n * 2.0 ** -23 * np.sum(np.abs(x.astype(np.float64)), axis=0)
    err = np.abs(g.astype(np.float64) - want.astype(np.float64))
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, f"atomic-order fp32 beyond bound at {bad[:8]}: err {err[bad[:8]]}"


def draw(dtype: str, n: int, count: int, seed: int, dist: str | None = None) -> np.ndarray:
    if dist is None:
        dist = {"f32": "uniform", "bf16": "normal", "i32": "int20"}[dtype]
    return I.rank_inputs(dist, dtype, n, count, workload=99, size_idx=seed, iteration=0)


def supports(algo: str, dtype: str) -> bool:
    return True


def elem_bytes(dtype: str) -> int:
    return I.ELEM_BYTES[dtype]


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [
    "ALGO_NAMES", "FIXED_ORDER", "assert_matches", "ceil_div", "draw", "elem_bytes",
    "from_device", "handle", "math", "oracle_sum", "run_allreduce", "supports", "to_device",
]
