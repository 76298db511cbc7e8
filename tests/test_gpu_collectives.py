"""GPU parity of the standalone reduce-scatter, all-gather and broadcast, through the C ABI,
against the CPU oracle's plain definitions. Every comparison is bit-exact: the reduce-scatter
folds in rank order like the AllReduce, and the other two move bytes."""

import numpy as np
import pytest

from tests.gpu_util import draw, elem_bytes, from_device, handle, to_device

pytestmark = pytest.mark.gpu

# partition sizes in elements: whole 16-byte units, one to several passes of a rank's lanes
PART_COUNTS = {"f32": [4, 12, 64, 1028, 17500], "i32": [4, 12, 64, 1028, 17500],
               "bf16": [8, 24, 1032, 17504, 35000]}
BCAST_COUNTS = [1, 3, 33, 1000, 4099, 70001]


def _say(*a):
    print(*a, flush=True)


def _np_dtype(x):
    return x.dtype


def _rows(x):
    return [np.ascontiguousarray(x[r]) for r in range(x.shape[0])]


def _same_bytes(got, want, what):
    g, w = got.view(np.uint8), np.ascontiguousarray(want).view(np.uint8)
    assert g.shape == w.shape, f"{what}: shape {g.shape} != {w.shape}"
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at byte {bad[:4]}"


def run_rs(h, x, n, inplace=False):
    from latency_collectives_amd import _ar as A
    import torch

    rc = x.shape[1] // n
    ins = to_device(x)
    if inplace:
        outs = [ins[r][r * rc:(r + 1) * rc] for r in range(n)]
    else:
        outs = [torch.full((rc,), 0x55, dtype=ins[0].dtype, device="cuda") for _ in range(n)]
    A.ar_reducescatter(h, ins, outs, rc)
    A.ar_check(h)
    return [o.cpu().numpy().view(x.dtype) for o in outs]


def run_ag(h, x, n, inplace=False):
    from latency_collectives_amd import _ar as A
    import torch

    sc = x.shape[1]
    dev = to_device(x)
    outs = [torch.full((n * sc,), 0x55, dtype=dev[0].dtype, device="cuda") for _ in range(n)]
    if inplace:
        for r in range(n):
            outs[r][r * sc:(r + 1) * sc].copy_(dev[r])
        ins = [outs[r][r * sc:(r + 1) * sc] for r in range(n)]
    else:
        ins = dev
    A.ar_allgather(h, ins, outs, sc)
    A.ar_check(h)
    return [o.cpu().numpy().view(x.dtype) for o in outs]


def run_bc(h, x, n, root, inplace=False):
    from latency_collectives_amd import _ar as A
    import torch

    dev = to_device(x[root:root + 1])[0]
    outs = [torch.full_like(dev, 0x55) for _ in range(n)]
    if inplace:
        outs[root] = dev
    A.ar_broadcast(h, dev, outs, x.shape[1], root)
    A.ar_check(h)
    return [o.cpu().numpy().view(x.dtype) for o in outs]


def check_rs(got, x, n):
    from oracle import oracle

    want = oracle.reducescatter(_rows(x))
    for r in range(n):
        _same_bytes(got[r], want[r], f"reduce-scatter rank {r}")


def check_ag(got, x, n):
    from oracle import oracle

    want = oracle.allgather(_rows(x))
    for r in range(n):
        _same_bytes(got[r], want[r], f"all-gather rank {r}")


def check_bc(got, x, n, root):
    from oracle import oracle

    want = oracle.broadcast(np.ascontiguousarray(x[root]), n)
    for r in range(n):
        _same_bytes(got[r], want[r], f"broadcast rank {r}")


# launch shapes: the planner's choice (one-pass halves of the two-shot kernel with 8- or 16-byte
# units where a chunk fits one pass, the loop kernels beyond), 16-byte units only, and one
# 64-thread workgroup per rank (every size but the smallest on the loop kernels)
SHAPES = {"auto": {}, "wide_units": {"narrow": 0}, "loop": {"ctas": 1, "threads": 64}}


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
def test_reducescatter_and_allgather(n, dtype, shape):
    counts = PART_COUNTS[dtype]
    with handle(n, n * max(counts) * elem_bytes(dtype), dtype, **SHAPES[shape]) as h:
        for i, c in enumerate(counts):
            _say(f"case reduce-scatter n={n} dtype={dtype} recvcount={c} shape={shape}")
            x = draw(dtype, n, n * c, seed=3000 + 10 * n + i)
            check_rs(run_rs(h, x, n), x, n)
            _say(f"case all-gather n={n} dtype={dtype} sendcount={c} shape={shape}")
            y = draw(dtype, n, c, seed=4000 + 10 * n + i)
            check_ag(run_ag(h, y, n), y, n)


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
def test_broadcast_every_root_kind(n, dtype, shape):
    with handle(n, max(BCAST_COUNTS) * elem_bytes(dtype), dtype, **SHAPES[shape]) as h:
        for i, c in enumerate(BCAST_COUNTS):
            for root in sorted({0, n // 2, n - 1}):
                _say(f"case broadcast n={n} dtype={dtype} count={c} root={root} shape={shape}")
                x = draw(dtype, n, c, seed=5000 + 10 * n + i)
                check_bc(run_bc(h, x, n, root), x, n, root)


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("n", [2, 4, 8])
def test_collectives_chunked_scratch(n, shape):
    """Scratch slots of 1 KiB: every call that does not fit the near slots is several chunks
    (several steps of one launch), the broadcast root waiting for its receivers' buffer flags
    from the third chunk on."""
    env = {"AR_SCRATCH_ONESHOT": 2048 * n, "AR_SCRATCH_TWOSHOT": 2048 * n}
    dtype = "f32"
    with handle(n, max(n * 1028, 3001) * 4, dtype, env=env, **SHAPES[shape]) as h:
        for it in range(2):
            _say(f"case chunked n={n} it={it} shape={shape}")
            x = draw(dtype, n, n * 1028, seed=6000 + it)
            check_rs(run_rs(h, x, n), x, n)
            y = draw(dtype, n, 1028, seed=6100 + it)
            check_ag(run_ag(h, y, n), y, n)
            z = draw(dtype, n, 3001, seed=6200 + it)
            check_bc(run_bc(h, z, n, n - 1), z, n, n - 1)


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("op", ["reducescatter", "allgather", "broadcast"])
@pytest.mark.parametrize("drift", [0, 3])
def test_collectives_persistent_loop(op, drift, shape):
    """ar_bench: 40 collectives in one launch over 8 input sets, with and without random rank
    drift; afterwards every set's output is checked (each set's last run wrote it)."""
    from latency_collectives_amd import _ar as A
    import torch

    n, dtype, c, iters, nsets = 4, "f32", 1028, 40, 8
    root = 2
    in_c = n * c if op == "reducescatter" else c
    out_c = n * c if op == "allgather" else c
    with handle(n, n * c * 4, dtype, drift=drift, root=root, **SHAPES[shape]) as h:
        xs = [draw(dtype, n, in_c, seed=7000 + k) for k in range(nsets)]
        ins, outs = [], []
        for x in xs:
            ins += to_device(x)
            outs += [torch.full((out_c,), 0x55, dtype=torch.float32, device="cuda")
                     for _ in range(n)]
        _say(f"case persistent {op} drift={drift} shape={shape}")
        ts, te, ms = A.ar_bench_ex(h, ins, outs, nsets, c, A.ALGOS[op], iters)
        assert ms > 0
        for k, x in enumerate(xs):
            got = [o.cpu().numpy() for o in outs[k * n:(k + 1) * n]]
            if op == "reducescatter":
                check_rs(got, x, n)
            elif op == "allgather":
                check_ag(got, x, n)
            else:
                check_bc(got, x, n, root)
        assert np.all(te.reshape(iters, n) >= ts.reshape(iters, n))


def test_collectives_in_place_and_rearmed():
    """The usual in-place forms give the same bytes, and every sentinel slot is armed again
    after the calls."""
    from latency_collectives_amd import _ar as A

    n, dtype, c = 4, "bf16", 1032
    with handle(n, n * c * 2, dtype) as h:
        for it in range(3):
            x = draw(dtype, n, n * c, seed=8000 + it)
            check_rs(run_rs(h, x, n, inplace=True), x, n)
            y = draw(dtype, n, c, seed=8100 + it)
            check_ag(run_ag(h, y, n, inplace=True), y, n)
            z = draw(dtype, n, 777, seed=8200 + it)
            check_bc(run_bc(h, z, n, 1, inplace=True), z, n, 1)
        for r in range(n):
            w = A.ar_read_region(h, r, A.REGION_P1).view(np.uint32)
            assert np.all(w == 0xFFFFFFFF), f"rank {r} slots not re-armed"


def test_collectives_argument_errors():
    from latency_collectives_amd import _ar as A
    import torch

    n = 2
    with handle(n, 4096, "f32") as h:
        a = [torch.zeros(2 * 6, device="cuda") for _ in range(n)]
        o = [torch.zeros(6, device="cuda") for _ in range(n)]
        with pytest.raises(A.ArError) as e:  # 6 fp32 = 24 bytes: not whole 16-byte units
            A.ar_reducescatter(h, a, o, 6)
        assert e.value.code == A.AR_EINVAL
        with pytest.raises(A.ArError) as e:
            A.ar_allgather(h, o, a, 6)
        assert e.value.code == A.AR_EINVAL
        big = [torch.zeros(4096, device="cuda") for _ in range(n)]
        with pytest.raises(A.ArError) as e:  # input 2 * 2048 fp32 > 4096 bytes
            A.ar_reducescatter(h, big, big, 1024)
        assert e.value.code == A.AR_ETOOBIG
        b = [torch.zeros(16, device="cuda") for _ in range(n)]
        with pytest.raises(A.ArError) as e:
            A.ar_broadcast(h, b[0], b, 16, 2)  # root out of range
        assert e.value.code == A.AR_EINVAL
        with pytest.raises(A.ArError) as e:
            A.ar_broadcast(h, b[0], [b[1], b[1]], 16, 0)  # outputs overlap
        assert e.value.code == A.AR_EINVAL
        x = [torch.zeros(2 * 8, device="cuda") for _ in range(n)]
        with pytest.raises(A.ArError) as e:  # output inside another rank's input
            A.ar_reducescatter(h, x, [x[1][:8], x[0][8:]], 8)
        assert e.value.code == A.AR_EINVAL
        e0 = A.ar_epoch(h)
        A.ar_reducescatter(h, x, o, 0)
        assert A.ar_epoch(h) == e0 + 1
        A.ar_check(h)


@pytest.mark.parametrize("op", ["reducescatter", "allgather", "broadcast"])
def test_collectives_withheld_rank_times_out(op):
    """Rank 0 (the broadcast root) sends nothing: the others' bounded polls give up, ar_check
    reports AR_ETIMEOUT and no wave is left running."""
    from latency_collectives_amd import _ar as A
    import torch

    n, c = 4, 1024
    with handle(n, n * c * 4, "f32", timeout_us=20000, withhold_rank=0) as h:
        x = draw("f32", n, n * c, seed=9)
        ins = to_device(x)
        if op == "reducescatter":
            A.ar_reducescatter(h, ins, [torch.empty(c, device="cuda") for _ in range(n)], c)
        elif op == "allgather":
            A.ar_allgather(h, [t[:c] for t in ins], [torch.empty(n * c, device="cuda")
                                                     for _ in range(n)], c)
        else:
            A.ar_broadcast(h, ins[0], [torch.empty(n * c, device="cuda") for _ in range(n)],
                           n * c, 0)
        with pytest.raises(A.ArError) as e:
            A.ar_check(h)
        assert e.value.code == A.AR_ETIMEOUT


def test_full_size_tp_decode_shapes():
    """8 ranks, bf16, the [tokens, 8192] decode activation at 64 tokens: reduce-scatter of the
    whole activation (output 64 x 1024 per rank), all-gather of a 64 x 1024 shard and broadcast
    of the whole activation, checked element by element."""
    n, dtype, t = 8, "bf16", 64
    with handle(n, t * 8192 * 2, dtype) as h:
        x = draw(dtype, n, t * 8192, seed=10, dist="normal")
        check_rs(run_rs(h, x, n), x, n)
        y = draw(dtype, n, t * 1024, seed=11, dist="normal")
        check_ag(run_ag(h, y, n), y, n)
        check_bc(run_bc(h, x, n, 5), x, n, 5)


def test_plan_info_reports_the_launch():
    """ar_plan_info describes the launch the calls make: the bulk two-shot with whole multiples
    of the rank's compute units as workgroups at 16 MiB, a near-region one-pass kernel for a
    small message, and the collectives' own kernels."""
    from latency_collectives_amd import _ar as A

    n = 8
    with handle(n, 16 << 20, "i32") as h:
        big = A.ar_plan_info(h, (16 << 20) // 4, A.AR_TWOSHOT)
        # 16 MiB two-shot cap: 1 MiB per (buffer, source) slot, so a 2 MiB partition is 2 chunks
        assert big["kernel"] == 7 and big["threads"] == 256 and big["chunks"] == 2
        # int32 sums may equal the sentinel: the int32 two-shot always runs the bulk kernel
        # (completion flags), on the regular slots, with one workgroup per 256 units when small
        small = A.ar_plan_info(h, 256, A.AR_TWOSHOT)
        assert small["kernel"] == 7 and small["near"] == 0 and small["chunks"] == 1
        assert small["ctas"] == 1
    with handle(n, 16 << 20, "f32") as hf:
        small_f = A.ar_plan_info(hf, 256, A.AR_TWOSHOT)
        assert small_f["kernel"] in (3, 11, 28, 29) and small_f["near"] == 1 and small_f["chunks"] == 1
        assert small_f["grid"] >= n * small_f["ctas"]
    with handle(n, 16 << 20, "i32") as h:
        rs = A.ar_plan_info(h, 1024, A.AR_REDUCESCATTER)
        ag = A.ar_plan_info(h, 1024, A.AR_ALLGATHER)
        bc = A.ar_plan_info(h, 1024, A.AR_BROADCAST)
        # one-pass kernels with 8-byte units on the near slots
        assert (rs["kernel"], ag["kernel"], bc["kernel"]) == (17, 18, 20)
        assert bc["near"] == 1
        assert rs["near"] == 1 and ag["near"] == 1 and rs["unit_bytes"] == 8
        for p in (big, small, rs, ag, bc):
            assert p["grid"] >= n * p["ctas"]
        import torch

        rank_cus = torch.cuda.get_device_properties(0).multi_processor_count // 8
        assert big["ctas"] % rank_cus == 0, (big, rank_cus)
        with pytest.raises(A.ArError) as e:
            A.ar_plan_info(h, 6, A.AR_REDUCESCATTER)  # 24 bytes: not whole units
        assert e.value.code == A.AR_EINVAL
        # a partition wider than one pass of the rank's lanes runs the loop kernels on regular slots
        wide_rs = A.ar_plan_info(h, (16 << 20) // 4 // n, A.AR_REDUCESCATTER)
        wide_ag = A.ar_plan_info(h, (16 << 20) // 4 // n, A.AR_ALLGATHER)
        wide_bc = A.ar_plan_info(h, (16 << 20) // 4, A.AR_BROADCAST)
        assert (wide_rs["kernel"], wide_ag["kernel"], wide_bc["kernel"]) == (12, 13, 14)
        assert wide_rs["near"] == 0 and wide_ag["near"] == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_pass_collectives_several_chunks(dtype):
    """8 ranks, 16 KiB slots: an 81 KiB partition misses the near slots but each 16 KiB chunk
    fits one pass, so the one-pass reduce-scatter runs six chunks per call, the last one short;
    all-gather and broadcast take their loop kernels on the regular slots, also in chunks."""
    from latency_collectives_amd import _ar as A

    n = 8
    env = {"AR_SCRATCH_ONESHOT": 2 * n * 16384, "AR_SCRATCH_TWOSHOT": 2 * n * 16384}
    part = 81 * 1024 // elem_bytes(dtype)
    bcount = 100003
    with handle(n, max(n * part * elem_bytes(dtype), bcount * elem_bytes(dtype)), dtype,
                env=env) as h:
        rs = A.ar_plan_info(h, part, A.AR_REDUCESCATTER)
        ag = A.ar_plan_info(h, part, A.AR_ALLGATHER)
        assert rs["kernel"] in (15, 17) and rs["chunks"] > 1 and rs["near"] == 0, rs
        assert ag["kernel"] == 13 and ag["chunks"] > 1 and ag["near"] == 0, ag
        for it in range(2):
            _say(f"case several chunks dtype={dtype} it={it}")
            x = draw(dtype, n, n * part, seed=9100 + it)
            check_rs(run_rs(h, x, n), x, n)
            y = draw(dtype, n, part, seed=9200 + it)
            check_ag(run_ag(h, y, n), y, n)
            z = draw(dtype, n, bcount, seed=9300 + it)
            check_bc(run_bc(h, z, n, 3), z, n, 3)


def test_every_algorithm_and_collective_interleaved_on_one_handle():
    """A seeded random sequence of AllReduces (every algorithm, near, regular and bulk sizes)
    and reduce-scatters, all-gathers and broadcasts on ONE handle, every result checked: the
    protocols share scratch regions (sentinel slots, near pages, the monotonic flag region that
    both the bulk two-shot and the broadcast credits use), so each call must leave them as the
    next one expects; persistent broadcast loops run after bulk two-shots."""
    from latency_collectives_amd import _ar as A
    from tests.gpu_util import assert_matches, run_allreduce

    n, dtype = 4, "f32"
    algos = ["auto", "oneshot_ll", "oneshot_sentinel", "twoshot", "ll128_atomic", "barrier2"]
    ar_counts = [5, 300, 4096, 70000, 600000]  # near, near, near, regular, bulk two-shot
    part_counts = [4, 256, 4100, 65536]
    g = np.random.default_rng(77)
    with handle(n, 600000 * 4, dtype) as h:
        for step in range(40):
            kind = g.integers(0, 4)
            seed = 12000 + step
            if kind == 0:
                algo = algos[g.integers(0, len(algos))]
                count = int(ar_counts[g.integers(0, len(ar_counts))])
                _say(f"case interleaved step={step} allreduce {algo} count={count}")
                x = draw(dtype, n, count, seed=seed)
                assert_matches(run_allreduce(h, x, algo), x, algo, dtype)
            elif kind == 1:
                c = int(part_counts[g.integers(0, len(part_counts))])
                _say(f"case interleaved step={step} reduce-scatter {c}")
                x = draw(dtype, n, n * c, seed=seed)
                check_rs(run_rs(h, x, n), x, n)
            elif kind == 2:
                c = int(part_counts[g.integers(0, len(part_counts))])
                _say(f"case interleaved step={step} all-gather {c}")
                x = draw(dtype, n, c, seed=seed)
                check_ag(run_ag(h, x, n), x, n)
            else:
                c = int(ar_counts[g.integers(0, len(ar_counts))])
                root = int(g.integers(0, n))
                _say(f"case interleaved step={step} broadcast {c} root={root}")
                x = draw(dtype, n, c, seed=seed)
                check_bc(run_bc(h, x, n, root), x, n, root)
        # a bulk two-shot, then a persistent broadcast loop (credit flags over the same region)
        x = draw(dtype, n, 600000, seed=13000)
        assert_matches(run_allreduce(h, x, "twoshot"), x, "twoshot", dtype)
        import torch

        A.ar_set_option(h, A.AR_OPT_ROOT, 1)
        for c in (300, 70000):
            xs = [draw(dtype, n, c, seed=13100 + c + k) for k in range(4)]
            ins, outs = [], []
            for xk in xs:
                ins += to_device(xk)
                outs += [torch.full((c,), 0x55, dtype=torch.float32, device="cuda")
                         for _ in range(n)]
            _say(f"case interleaved persistent broadcast count={c}")
            A.ar_bench(h, ins, outs, 4, c, A.AR_BROADCAST, 20, timestamps=False)
            for k, xk in enumerate(xs):
                check_bc([o.cpu().numpy() for o in outs[k * n:(k + 1) * n]], xk, n, 1)
        for r in range(n):
            for reg in (A.REGION_P1, A.REGION_P2, A.REGION_P1_NEAR, A.REGION_P2_NEAR):
                w = A.ar_read_region(h, r, reg).view(np.uint32)
                assert np.all(w == 0xFFFFFFFF), f"rank {r} region {reg} not re-armed"
