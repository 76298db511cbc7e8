"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers; it holds none of the AllReduce arithmetic. Both the GPU path and
the CPU oracle are fed from here, so neither side generates its own data.

Recipe. Every (workload, size index, iteration, rank) gets its own stream,
``numpy.random.Generator(PCG64(SeedSequence([workload, size_idx, iteration, rank])))``, so an
input can be regenerated on its own without replaying the others. Distributions:

* ``uniform``   : binary32 uniform on [-1, 1)  (drawn as float64, then rounded to binary32).
* ``normal``    : normal(0, sigma) drawn as binary32, then rounded to bfloat16 with torch's
                  round-to-nearest-even conversion; every value is checked to be finite.
* ``int20``     : int32 uniform on [-2**20, 2**20], both ends included.
* ``dyadic``    : k * 2**-10 with k uniform on [-2**10, 2**10]; any sum of up to 16 of them is
                  exact in binary32, whatever the order of the additions.
* ``rankconst`` : rank r is filled with the constant r.

bfloat16 values are returned as ``numpy.uint16`` bit patterns.
"""

from __future__ import annotations

import numpy as np

BF16 = "bf16"
F32 = "f32"
I32 = "i32"

NP_DTYPE = {F32: np.float32, BF16: np.uint16, I32: np.int32}
ELEM_BYTES = {F32: 4, BF16: 2, I32: 4}


def _rng(workload: int, size_idx: int, iteration: int, rank: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(workload), int(size_idx), int(iteration), int(rank)])
    return np.random.Generator(np.random.PCG64(ss))


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch  # only for its float32 -> bfloat16 conversion (round to nearest even)

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw(dist: str, dtype: str, count: int, workload: int, size_idx: int, iteration: int,
         rank: int, sigma: float = 1.0) -> np.ndarray:
    """One rank's input: ``count`` elements of ``dtype`` from distribution ``dist``."""
    g = _rng(workload, size_idx, iteration, rank)
    if dist == "rankconst":
        if dtype == BF16:
            return _to_bf16_bits(np.full(count, float(rank), np.float32))
        return np.full(count, rank, dtype=NP_DTYPE[dtype])
    if dist == "uniform":
        if dtype != F32:
            raise ValueError("uniform inputs are binary32")
        return g.uniform(-1.0, 1.0, count).astype(np.float32)
    if dist == "dyadic":
        k = g.integers(-(1 << 10), 1 << 10, size=count, endpoint=True)
        if dtype == F32:
            return (k.astype(np.float64) / 1024.0).astype(np.float32)
        if dtype == I32:
            return k.astype(np.int32)
        raise ValueError("dyadic inputs are binary32 or int32")
    if dist == "normal":
        x = g.standard_normal(count, dtype=np.float32) * np.float32(sigma)
        if dtype == F32:
            out = x.astype(np.float32)
        elif dtype == BF16:
            out = _to_bf16_bits(x)
        else:
            raise ValueError("normal inputs are binary32 or bfloat16")
        return out
    if dist == "int20":
        if dtype != I32:
            raise ValueError("int20 inputs are int32")
        return g.integers(-(1 << 20), 1 << 20, size=count, endpoint=True).astype(np.int32)
    raise ValueError(f"unknown distribution {dist!r}")


def rank_inputs(dist: str, dtype: str, nranks: int, count: int, workload: int, size_idx: int,
                iteration: int, sigma: float = 1.0) -> np.ndarray:
    """All ranks' inputs for one iteration, shape [nranks, count]."""
    out = np.empty((nranks, count), dtype=NP_DTYPE[dtype])
    for r in range(nranks):
        out[r] = draw(dist, dtype, count, workload, size_idx, iteration, r, sigma)
    return out


def assert_finite(x: np.ndarray, dtype: str) -> None:
    """Raise if a floating-point input holds a NaN or an infinity (inputs must be finite)."""
    if dtype == F32:
        ok = np.isfinite(x).all()
    elif dtype == BF16:
        ok = ((x.astype(np.uint32) & 0x7F80) != 0x7F80).all()
    else:
        ok = True
    if not ok:
        raise ValueError("non-finite input drawn")


# The five workloads the benchmark and the parity tests use. Sizes are bytes per rank.
WORKLOADS = {
    1: dict(name="oneshot_ll_n2_f32_128B", nranks=2, dtype=F32, dist="uniform", sigma=1.0,
            sizes=[128], iters=1000, algo="oneshot_ll"),
    2: dict(name="oneshot_sentinel_n4_bf16_1K-256K", nranks=4, dtype=BF16, dist="normal",
            sigma=1.0, sizes=[1 << k for k in range(10, 19)], iters=200,
            algo="oneshot_sentinel"),
    3: dict(name="twoshot_n8_bf16_tp_decode_8192", nranks=8, dtype=BF16, dist="normal",
            sigma=0.5, sizes=[t * 8192 * 2 for t in (1, 2, 4, 8, 16, 32, 64)], iters=100,
            algo="twoshot"),
    4: dict(name="ll128_vs_oneshot_vs_barrier_n16_f32_4K-4M", nranks=16, dtype=F32,
            dist="uniform", sigma=1.0, sizes=[1 << k for k in range(12, 23)], iters=100,
            algo="ll128_atomic"),
    5: dict(name="twoshot_n8_bandwidth_16M-256M", nranks=8, dtype=I32, dist="int20", sigma=1.0,
            sizes=[1 << k for k in range(24, 29)], iters=20, algo="twoshot"),
    # the standalone collectives on the same decode activation [tokens, 8192] bf16 at 8 ranks;
    # sizes are the per-rank partition: the reduce-scatter output [t, 1024], the all-gather
    # input [t, 1024], the whole broadcast activation [t, 8192]
    6: dict(name="reducescatter_n8_bf16_tp_decode_8192", nranks=8, dtype=BF16, dist="normal",
            sigma=0.5, sizes=[t * 1024 * 2 for t in (1, 2, 4, 8, 16, 32, 64)], iters=100,
            algo="reducescatter"),
    7: dict(name="allgather_n8_bf16_tp_decode_8192", nranks=8, dtype=BF16, dist="normal",
            sigma=0.5, sizes=[t * 1024 * 2 for t in (1, 2, 4, 8, 16, 32, 64)], iters=100,
            algo="allgather"),
    8: dict(name="broadcast_n8_bf16_tp_decode_8192", nranks=8, dtype=BF16, dist="normal",
            sigma=0.5, sizes=[t * 8192 * 2 for t in (1, 2, 4, 8, 16, 32, 64)], iters=100,
            algo="broadcast"),
}
COLLECTIVES = ("reducescatter", "allgather", "broadcast")


def device_draw(dist: str, dtype: str, nranks: int, count: int, workload: int, size_idx: int,
                iteration: int, sigma: float = 1.0):
    """Like :func:`rank_inputs` but drawn on the GPU with a seeded torch generator (for
    messages too large to generate on the host quickly). Returns a list of nranks device
    tensors (bfloat16 data as int16 bit patterns). The stream differs from the host recipe."""
    import torch

    seed = int(np.random.SeedSequence([workload, size_idx, iteration, 1 << 20]).generate_state(1)[0])
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for r in range(nranks):
        if dist == "rankconst":
            t = torch.full((count,), r, device="cuda",
                           dtype={F32: torch.float32, I32: torch.int32, BF16: torch.float32}[dtype])
            if dtype == BF16:
                t = t.to(torch.bfloat16).view(torch.int16)
        elif dist == "uniform":
            t = torch.rand(count, generator=g, device="cuda", dtype=torch.float32) * 2.0 - 1.0
        elif dist == "int20":
            t = torch.randint(-(1 << 20), (1 << 20) + 1, (count,), generator=g, device="cuda",
                              dtype=torch.int32)
        elif dist == "normal":
            t = torch.randn(count, generator=g, device="cuda", dtype=torch.float32) * sigma
            if dtype == BF16:
                t = t.to(torch.bfloat16).view(torch.int16)
        else:
            raise ValueError(f"no device recipe for {dist!r}")
        out.append(t.contiguous())
    return out
