"""Pins for the CPU oracle (no GPU).

The oracle is only trusted because these tests tie it to facts that do not come from the oracle:
hand-worked golden cases, closed forms, exact integer arithmetic done by Python, library
conversions and IEEE addition done by numpy, and error bounds of recursive summation. Each test
names the kind of mistake it would catch.
"""

import itertools
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


# ---------------------------------------------------------------- invariants and closed forms

@pytest.mark.parametrize("n", list(range(1, 17)))
@pytest.mark.parametrize("dt", [np.float32, np.int32, np.float64])
def test_rank_constant_closed_form(oracle_mod, n, dt):
    """Rank r filled with r sums to N(N-1)/2 everywhere, and all ranks agree (a dropped or
    doubled rank, or an off-by-one in the rank loop, breaks the closed form)."""
    count = 37
    x = [np.full(count, r, dtype=dt) for r in range(n)]
    out = oracle_mod.allreduce(x)
    for o in out:
        assert np.array_equal(o, np.full(count, n * (n - 1) // 2, dtype=dt))


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16])
def test_rank_constant_bf16(oracle_mod, n):
    """bf16 inputs r (exact) sum to N(N-1)/2, which is exact in bf16 for N <= 16 (<= 120)."""
    import torch

    count = 19
    x = [torch.full((count,), float(r)).to(torch.bfloat16).view(torch.int16).numpy()
         .view(np.uint16).copy() for r in range(n)]
    out = oracle_mod.allreduce(x)
    want = torch.full((count,), float(n * (n - 1) // 2)).to(torch.bfloat16).view(torch.int16)
    for o in out:
        assert np.array_equal(o, want.numpy().view(np.uint16))


@pytest.mark.parametrize("dt", [np.float32, np.int32, np.float64, np.uint16])
def test_single_rank_is_copy(oracle_mod, dt):
    """N = 1 returns the input bit for bit (special values included for the float types)."""
    g = np.random.default_rng(1)
    if dt == np.uint16:
        x = g.integers(0, 1 << 16, size=257).astype(np.uint16)
        x = x[((x & 0x7F80) != 0x7F80)]  # finite bf16 only: NaN payloads are not preserved
    elif dt == np.int32:
        x = g.integers(-(1 << 31), 1 << 31, size=257).astype(np.int32)
    else:
        x = g.standard_normal(257).astype(dt)
        x[:4] = [0.0, -0.0, np.inf, -np.inf]
    x = np.ascontiguousarray(x)
    out = oracle_mod.allreduce([x])[0]
    assert np.array_equal(out.view(np.uint8), x.view(np.uint8))


def test_two_rank_fp32_is_ieee_sum(oracle_mod):
    """N = 2 in binary32 is one IEEE addition, which is commutative; numpy's float32 add is an
    independent implementation of it (a wrong rounding mode or a wider accumulator fails)."""
    g = np.random.default_rng(2)
    a = (g.standard_normal(4096) * 10.0 ** g.integers(-6, 6, 4096)).astype(np.float32)
    b = (g.standard_normal(4096) * 10.0 ** g.integers(-6, 6, 4096)).astype(np.float32)
    out = oracle_mod.allreduce([a, b])
    want = a + b
    assert np.array_equal(out[0].view(np.uint32), want.view(np.uint32))
    assert np.array_equal(out[1].view(np.uint32), want.view(np.uint32))
    swapped = oracle_mod.allreduce([b, a])[0]
    assert np.array_equal(swapped.view(np.uint32), want.view(np.uint32))


def test_outputs_identical_across_ranks(oracle_mod):
    g = np.random.default_rng(3)
    for n in (2, 3, 8, 16):
        x = [g.uniform(-1, 1, 1000).astype(np.float32) for _ in range(n)]
        out = oracle_mod.allreduce(x)
        for o in out[1:]:
            assert np.array_equal(o.view(np.uint32), out[0].view(np.uint32))


# ---------------------------------------------------------------- exact integer arithmetic

@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_int_brute_force_small_range(oracle_mod, n):
    """Every combination of per-rank values in {-2..2}, one combination per element, against
    Python's exact integer sum (catches a dropped term, a sign slip or a wrong index)."""
    combos = list(itertools.product(range(-2, 3), repeat=n))
    x = [np.array([c[r] for c in combos], dtype=np.int32) for r in range(n)]
    out = oracle_mod.allreduce(x)
    want = np.array([sum(c) for c in combos], dtype=np.int32)
    for o in out:
        assert np.array_equal(o, want)


@pytest.mark.parametrize("count", [1, 2, 3])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_int_brute_force_counts(oracle_mod, n, count):
    """Tiny counts, every element distinct: element i of the output only sees element i."""
    g = np.random.default_rng(n * 10 + count)
    x = [g.integers(-2, 3, size=count).astype(np.int32) for _ in range(n)]
    out = oracle_mod.allreduce(x)
    want = [sum(int(x[r][i]) for r in range(n)) for i in range(count)]
    for o in out:
        assert o.tolist() == want


def test_int_large_random_vs_python(oracle_mod):
    """Config-5-like int32 inputs in [-2^20, 2^20] at N = 8, against numpy int64 sums."""
    g = np.random.default_rng(5)
    x = [g.integers(-(1 << 20), 1 << 20, size=10000, endpoint=True).astype(np.int32)
         for _ in range(8)]
    out = oracle_mod.allreduce(x)
    want = np.sum(np.stack(x).astype(np.int64), axis=0)
    assert np.array_equal(out[0].astype(np.int64), want)


def test_golden_int(oracle_mod):
    for ln in _lines("allreduce_small_i32.txt"):
        lhs, rhs = ln.split(";")
        ranks = [np.array([int(v) for v in part.split()], dtype=np.int32)
                 for part in lhs.split("|")]
        want = np.array([int(v) for v in rhs.split()], dtype=np.int32)
        out = oracle_mod.allreduce(ranks)
        for o in out:
            assert np.array_equal(o, want), ln


def test_count_zero_is_noop(oracle_mod):
    x = [np.zeros(0, np.float32), np.zeros(0, np.float32)]
    out = oracle_mod.allreduce(x)
    assert all(o.size == 0 for o in out)


def test_in_place(oracle_mod):
    g = np.random.default_rng(6)
    x = [g.uniform(-1, 1, 333).astype(np.float32) for _ in range(4)]
    want = oracle_mod.allreduce([a.copy() for a in x])[0]
    oracle_mod.allreduce(x, out=x)
    for a in x:
        assert np.array_equal(a.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- binary32 fold order

def test_golden_fold_order(oracle_mod):
    """Hand-worked binary32 cases whose result depends on the addition order: pins the left
    fold over ranks 0..N-1 (a reversed, pairwise or own-rank-first order fails)."""
    for ln in _lines("fold_order_f32.txt"):
        lhs, rhs = ln.split(";")
        vals = [float(v) for v in lhs.split()]
        ranks = [np.array([v], dtype=np.float32) for v in vals]
        assert all(float(r[0]) == v for r, v in zip(ranks, vals))  # exact inputs
        out = oracle_mod.allreduce(ranks)
        for o in out:
            assert float(o[0]) == float(rhs), ln


def test_fold_matches_numpy_sequential_float32(oracle_mod):
    """The fold is a chain of binary32 additions in rank order: numpy's float32 add applied in
    the same order is an independent implementation of each step."""
    g = np.random.default_rng(7)
    n = 16
    x = [(g.standard_normal(2000) * 10.0 ** g.integers(-3, 4, 2000)).astype(np.float32)
         for _ in range(n)]
    acc = x[0].copy()
    for q in range(1, n):
        acc = (acc + x[q]).astype(np.float32)
    out = oracle_mod.allreduce(x)[0]
    assert np.array_equal(out.view(np.uint32), acc.view(np.uint32))


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_fp32_within_recursive_summation_bound(oracle_mod, n):
    """|fold - exact| <= (N-1) u sum|x| (u = 2^-24): the standard bound for recursive summation.
    The exact sum comes from math.fsum on the binary32 values (a wrong accumulator width or a
    dropped term breaks it)."""
    g = np.random.default_rng(8 + n)
    count = 3000
    x = [g.uniform(-1, 1, count).astype(np.float32) for _ in range(n)]
    out = oracle_mod.allreduce(x)[0].astype(np.float64)
    u = 2.0 ** -24
    for i in range(count):
        col = [float(x[r][i]) for r in range(n)]
        exact = math.fsum(col)
        bound = (n - 1) * u * sum(abs(v) for v in col) / (1 - (n - 1) * u)
        assert abs(out[i] - exact) <= bound


@pytest.mark.parametrize("n", [2, 5, 16])
def test_dyadic_exact_any_order(oracle_mod, n):
    """Inputs k * 2^-10 with |k| <= 2^10: every partial sum of <= 16 terms is exact in binary32,
    so the fold equals the exact sum computed with Python integers."""
    g = np.random.default_rng(9 + n)
    k = g.integers(-(1 << 10), 1 << 10, size=(n, 4096), endpoint=True)
    x = [(k[r] / 1024.0).astype(np.float32) for r in range(n)]
    out = oracle_mod.allreduce(x)[0]
    want = k.sum(axis=0) / 1024.0
    assert np.array_equal(out.astype(np.float64), want)


def test_f64_oracle_close_to_fsum(oracle_mod):
    g = np.random.default_rng(10)
    x = [g.uniform(-1, 1, 500) for _ in range(16)]
    out = oracle_mod.allreduce(x)[0]
    for i in range(500):
        exact = math.fsum(float(x[r][i]) for r in range(16))
        assert abs(out[i] - exact) <= 15 * 2.0 ** -53 * sum(abs(x[r][i]) for r in range(16)) * 1.01


# ---------------------------------------------------------------- bfloat16

def test_golden_bf16_rounding(oracle_mod):
    L = oracle_mod.lib()
    for ln in _lines("bf16_rounding.txt"):
        src, want = [p.strip() for p in ln.split(";")[:2]]
        f = np.array([int(src, 16)], dtype=np.uint32).view(np.float32)[0]
        assert L.oracle_f32_to_bf16(float(f)) == int(want, 16), ln


def test_bf16_conversion_matches_torch(oracle_mod):
    """torch's float32 -> bfloat16 conversion is round-to-nearest-even; on random values, on
    constructed exact ties and on values one ulp off ties the two must agree bit for bit."""
    import torch

    g = np.random.default_rng(11)
    vals = (g.standard_normal(3000) * 10.0 ** g.integers(-30, 30, 3000)).astype(np.float32)
    bits = g.integers(0, 1 << 31, size=3000).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]  # finite
    ties = (bits & 0xFFFF0000) | 0x8000
    near = np.concatenate([ties - 1, ties + 1]).astype(np.uint32)
    allv = np.concatenate([vals.view(np.uint32), bits, ties, near]).astype(np.uint32)
    f = allv.view(np.float32)
    f = f[np.isfinite(f)]
    mine = oracle_mod.f32_to_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_widen_exact(oracle_mod):
    """bf16 -> binary32 is exact: widening every finite bf16 pattern and narrowing back gives the
    same pattern."""
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    b = b[((b & 0x7F80) != 0x7F80)][::7]
    f = oracle_mod.bf16_to_f32(b)
    assert np.array_equal(oracle_mod.f32_to_bf16(f), b)


def test_golden_bf16_allreduce(oracle_mod):
    """Pins "fold in binary32, round once at the end" (rounding after every addition fails the
    third case; no rounding at all cannot produce a bf16 pattern)."""
    for ln in _lines("bf16_allreduce.txt"):
        lhs, rhs = [p.strip() for p in ln.split(";")[:2]]
        ranks = [np.array([int(v, 16)], dtype=np.uint16) for v in lhs.split("|")]
        out = oracle_mod.allreduce(ranks)
        for o in out:
            assert int(o[0]) == int(rhs, 16), ln


def test_bf16_allreduce_vs_float64_then_round(oracle_mod):
    """bf16 fold against an independent route: widen with a numpy bit shift, sum in float64,
    and require the oracle's bf16 result within one bf16 ulp of that near-exact sum (half an
    ulp from the final rounding plus the tiny binary32 fold error)."""
    import torch

    g = np.random.default_rng(12)
    n, count = 8, 4000
    src = g.standard_normal((n, count)).astype(np.float32)
    xb = torch.from_numpy(src).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ranks = [np.ascontiguousarray(xb[r]) for r in range(n)]
    out = oracle_mod.allreduce(ranks)[0]
    wide = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = wide.sum(axis=0)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ulp = np.array([2.0 ** (math.floor(math.log2(abs(v))) - 7) if v != 0 else 2.0 ** -133
                    for v in exact])
    # one bf16 rounding (half an ulp) plus the binary32 fold error, far below an ulp here
    assert np.all(np.abs(got - exact) <= ulp)


# ---------------------------------------------------------------- grouped (deterministic atomic) fold

def test_golden_grouped_fold(oracle_mod):
    """Hand-worked cases of the hierarchical order (groups of G consecutive ranks in rank order,
    then the group sums in group order): the same inputs give different binary32 results for
    G = 1, 2, 3, so a wrong group boundary, a dropped short last group or a plain left fold
    fails one of them."""
    for ln in _lines("grouped_fold.txt"):
        dt, grp, lhs, rhs = [p.strip() for p in ln.split(";")[:4]]
        if dt == "f32":
            vals = [float(v) for v in lhs.split()]
            ranks = [np.array([v], dtype=np.float32) for v in vals]
            assert all(float(r[0]) == v for r, v in zip(ranks, vals))  # exact inputs
            out = oracle_mod.allreduce_grouped(ranks, int(grp))
            for o in out:
                assert float(o[0]) == float(rhs), ln
        else:
            ranks = [np.array([int(v, 16)], dtype=np.uint16) for v in lhs.split()]
            out = oracle_mod.allreduce_grouped(ranks, int(grp))
            for o in out:
                assert int(o[0]) == int(rhs, 16), ln


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 16])
def test_grouped_fold_special_cases_are_the_left_fold(oracle_mod, n):
    """G = 1 and G >= N reduce to the plain left fold (pinned above), for fp32 and bf16."""
    import torch

    g = np.random.default_rng(40 + n)
    x = [g.standard_normal(777).astype(np.float32) * np.float32(10.0 ** g.integers(-2, 3))
         for _ in range(n)]
    want = oracle_mod.allreduce(x)[0]
    for grp in (1, n, n + 3):
        got = oracle_mod.allreduce_grouped(x, grp)[0]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), grp
    xb = [torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
          for a in x]
    wantb = oracle_mod.allreduce(xb)[0]
    for grp in (1, n):
        assert np.array_equal(oracle_mod.allreduce_grouped(xb, grp)[0], wantb), grp


@pytest.mark.parametrize("n,grp", [(4, 2), (8, 3), (16, 4), (16, 5)])
def test_grouped_fold_closed_forms_and_exactness(oracle_mod, n, grp):
    """Rank r filled with r sums to N(N-1)/2 in any order; dyadic inputs k * 2^-10 have exact
    partial sums, so the grouped fold equals the integer sum; every rank's output is the same."""
    x = [np.full(100, r, dtype=np.float32) for r in range(n)]
    out = oracle_mod.allreduce_grouped(x, grp)
    for o in out:
        assert np.all(o == n * (n - 1) / 2)
    g = np.random.default_rng(50 + n + grp)
    k = g.integers(-(1 << 10), 1 << 10, size=(n, 2048), endpoint=True)
    xd = [(k[r] / 1024.0).astype(np.float32) for r in range(n)]
    got = oracle_mod.allreduce_grouped(xd, grp)[0]
    assert np.array_equal(got.astype(np.float64), k.sum(axis=0) / 1024.0)


@pytest.mark.parametrize("n,grp", [(8, 4), (16, 4), (16, 2)])
def test_grouped_fold_within_its_summation_bound(oracle_mod, n, grp):
    """Error against math.fsum within the recursive-summation bound of the grouped order: a term
    passes through at most (G - 1) group additions and (ceil(N / G) - 1) group-sum additions,
    each with unit roundoff u = 2^-24."""
    g = np.random.default_rng(60 + n + grp)
    count = 2000
    x = [g.uniform(-1, 1, count).astype(np.float32) for _ in range(n)]
    out = oracle_mod.allreduce_grouped(x, grp)[0].astype(np.float64)
    steps = (grp - 1) + (-(-n // grp) - 1)
    u = 2.0 ** -24
    for i in range(count):
        col = [float(x[r][i]) for r in range(n)]
        bound = steps * u * sum(abs(v) for v in col) / (1 - steps * u)
        assert abs(out[i] - math.fsum(col)) <= bound


# ---------------------------------------------------------------- standalone collectives
#
# Reduce-scatter, all-gather and broadcast have no printed worked example on the pages; they are
# pinned by the decomposition the paper cites (an all-gather of a reduce-scatter is the
# AllReduce, itself pinned above), by integer arithmetic done in numpy with an independent
# formula, and by tagged inputs whose positions can be decoded.

def _rand_rows(g, n, count, dt):
    if dt == np.int32:
        return [g.integers(-(1 << 20), (1 << 20) + 1, size=count).astype(np.int32) for _ in range(n)]
    if dt == np.uint16:
        import torch
        return [torch.from_numpy(g.normal(size=count).astype(np.float32)).to(torch.bfloat16)
                .view(torch.int16).numpy().view(np.uint16).copy() for _ in range(n)]
    return [g.uniform(-1, 1, size=count).astype(dt) for _ in range(n)]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("dt", [np.float32, np.uint16, np.int32, np.float64])
def test_allgather_of_reducescatter_is_allreduce(oracle_mod, n, dt):
    """The decomposition AllReduce = AllGather(ReduceScatter) holds bit for bit (a wrong
    partition index, a transposed rank/partition loop or a different fold order breaks it)."""
    g = np.random.default_rng(100 + n)
    rc = 13
    x = _rand_rows(g, n, n * rc, dt)
    rs = oracle_mod.reducescatter(x)
    ag = oracle_mod.allgather(rs)
    ar = oracle_mod.allreduce(x)
    for r in range(n):
        assert rs[r].size == rc
        assert np.array_equal(ag[r].view(np.uint8), ar[r].view(np.uint8))


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("rc", [1, 2, 3])
def test_reducescatter_int_brute_force(oracle_mod, n, rc):
    """Small integer inputs against numpy's column sums of the [rank, partition, element] view
    (an independent formula: exact integer arithmetic, no fold)."""
    g = np.random.default_rng(7 * n + rc)
    for _ in range(20):
        x = g.integers(-2, 3, size=(n, n * rc)).astype(np.int32)
        got = oracle_mod.reducescatter([x[q].copy() for q in range(n)])
        want = x.reshape(n, n, rc).astype(np.int64).sum(axis=0)
        for r in range(n):
            assert np.array_equal(got[r].astype(np.int64), want[r])


@pytest.mark.parametrize("n", [2, 5, 16])
def test_reducescatter_rank_constant(oracle_mod, n):
    """Rank q filled with q: every element of every output is N(N-1)/2."""
    x = [np.full(n * 9, q, dtype=np.float32) for q in range(n)]
    for o in oracle_mod.reducescatter(x):
        assert np.array_equal(o, np.full(9, n * (n - 1) // 2, dtype=np.float32))


@pytest.mark.parametrize("n", [1, 2, 3, 8, 16])
def test_allgather_tagged_positions(oracle_mod, n):
    """Element i of rank q's input carries q * 100000 + i; in every output, position
    q * count + i must decode back to (q, i)."""
    count = 37
    x = [(q * 100000 + np.arange(count)).astype(np.int32) for q in range(n)]
    for o in oracle_mod.allgather(x):
        assert o.size == n * count
        pos = np.arange(n * count)
        assert np.array_equal(o // 100000, pos // count)
        assert np.array_equal(o % 100000, pos % count)


@pytest.mark.parametrize("dt", [np.uint16, np.float32])
def test_allgather_single_rank_and_bytes(oracle_mod, dt):
    """N = 1 is a copy; every byte pattern (NaNs included) passes through untouched."""
    g = np.random.default_rng(3)
    raw = g.integers(0, 256, size=64 * np.dtype(dt).itemsize).astype(np.uint8)
    x = raw.view(dt).copy()
    assert np.array_equal(oracle_mod.allgather([x])[0].view(np.uint8), raw)


@pytest.mark.parametrize("n", [1, 2, 7, 16])
def test_broadcast_copies_root(oracle_mod, n):
    """Every output equals the root's input byte for byte, for any byte pattern."""
    g = np.random.default_rng(n)
    root = g.integers(0, 256, size=1001).astype(np.uint8)
    outs = oracle_mod.broadcast(root, n)
    assert len(outs) == n
    for o in outs:
        assert np.array_equal(o, root)


@pytest.mark.parametrize("n", [2, 3, 5, 8, 16])
def test_int_rank_permutation_invariance(oracle_mod, n):
    """Integer sums are exact, so permuting which rank holds which input must not change any
    output bit (a dropped, doubled or mis-indexed rank would change the sum for some order)."""
    g = np.random.default_rng(500 + n)
    x = [g.integers(-(1 << 20), (1 << 20) + 1, size=333).astype(np.int32) for _ in range(n)]
    want = oracle_mod.allreduce(x)[0]
    for _ in range(5):
        perm = g.permutation(n)
        got = oracle_mod.allreduce([x[p] for p in perm])
        for o in got:
            assert np.array_equal(o, want)
    rs_want = oracle_mod.reducescatter([np.tile(a, n) for a in x])
    perm = g.permutation(n)
    rs_got = oracle_mod.reducescatter([np.tile(x[p], n) for p in perm])
    for a, b in zip(rs_got, rs_want):
        assert np.array_equal(a, b)
