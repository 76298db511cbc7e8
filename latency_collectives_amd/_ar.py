"""ctypes binding of the C ABI in ``include/ar.h`` (argument marshalling only).

Every function here has the name of the C entry point it wraps and does no computation of its
own: device pointers may be given as integers or as torch tensors (their ``data_ptr()``),
streams as integers, ``torch.cuda.Stream`` objects or ``None`` (torch's current stream).
A failing call raises :class:`ArError` carrying the C return code and ``ar_last_error()``.
The library must have been built (``python -m latency_collectives_amd.build``); loading fails
loudly otherwise: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libar.so")

AR_FLOAT32, AR_BFLOAT16, AR_INT32 = 0, 1, 2
(AR_ALGO_AUTO, AR_ONESHOT_LL, AR_ONESHOT_SENTINEL, AR_TWOSHOT, AR_LL128_ATOMIC, AR_BARRIER2,
 AR_BARRIER_ONLY) = range(7)
AR_REDUCESCATTER, AR_ALLGATHER, AR_BROADCAST = 12, 13, 14
AR_LL128_DET = 21
AR_OK, AR_EINVAL, AR_ETOOBIG, AR_ENOTSUP, AR_EHIP, AR_ETIMEOUT, AR_ENORES = 0, -1, -2, -3, -4, -5, -6
AR_PLACE_XCD, AR_PLACE_SAME, AR_PLACE_LINEAR = 0, 1, 2
(AR_OPT_TIMEOUT_US, AR_OPT_WITHHOLD_RANK, AR_OPT_CTAS, AR_OPT_THREADS, AR_OPT_PLACEMENT,
 AR_OPT_DRIFT, AR_OPT_NARROW, AR_OPT_ROOT, AR_OPT_CHECK_INPUTS, AR_OPT_RECORD_LAUNCH,
 AR_OPT_GROUP, AR_OPT_COOPERATIVE, AR_OPT_SPLIT, AR_OPT_TWO_HALVES, AR_OPT_TWO_PAGE) = range(15)
(REGION_P1, REGION_P2, REGION_LL, REGION_ACC, REGION_CNT, REGION_BAR, REGION_BDAT,
 REGION_LL_NEAR, REGION_P1_NEAR, REGION_P2_NEAR, REGION_PF1, REGION_PF2, REGION_FLG,
 REGION_LAUNCH_RECORD, REGION_SINK) = range(15)

ALGOS = {
    "auto": AR_ALGO_AUTO,
    "oneshot_ll": AR_ONESHOT_LL,
    "oneshot_sentinel": AR_ONESHOT_SENTINEL,
    "twoshot": AR_TWOSHOT,
    "ll128_atomic": AR_LL128_ATOMIC,
    "ll128_det": AR_LL128_DET,
    "barrier2": AR_BARRIER2,
    "barrier_only": AR_BARRIER_ONLY,
    "reducescatter": AR_REDUCESCATTER,
    "allgather": AR_ALLGATHER,
    "broadcast": AR_BROADCAST,
}
DTYPES = {"f32": AR_FLOAT32, "bf16": AR_BFLOAT16, "i32": AR_INT32}

# Every symbol include/ar.h declares.
EXPORTS = (
    "ar_create", "ar_allreduce", "ar_allreduce_noalloc", "ar_reducescatter", "ar_allgather", "ar_broadcast",
    "ar_destroy", "ar_last_error", "ar_check", "ar_bench", "ar_bench_ex",
    "ar_wallclock_hz", "ar_set_option", "ar_region_bytes", "ar_alg_bytes", "ar_plan_info",
    "ar_read_region",
    "ar_epoch",
    "ar_sol", "ar_sol_ex", "ar_sol_ranks", "ar_pingpong", "ar_torn_lines", "ar_stream_copy",
)


class ArError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class ar_plan(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in
                ("kernel", "chunks", "ctas", "threads", "grid", "unit_bytes", "near",
                 "resident_per_cu", "cu_count")]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class ar_sol_result(ctypes.Structure):
    _fields_ = [
        ("fence_ns", ctypes.c_double),
        ("l2_load_ns", ctypes.c_double),
        ("coherent_load_ns", ctypes.c_double),
        ("mall_load_ns", ctypes.c_double),
        ("hbm_load_ns", ctypes.c_double),
        ("store_half_rtt_ns", ctypes.c_double),
        ("store_half_rtt_far_ns", ctypes.c_double),
        ("floor_ns", ctypes.c_double),
        ("floor_fence_ns", ctypes.c_double),
        ("xcc_a", ctypes.c_int),
        ("xcc_b", ctypes.c_int),
    ]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class ar_sol_ranks_result(ctypes.Structure):
    _fields_ = [
        ("store_half_rtt_worst_ns", ctypes.c_double),
        ("store_half_rtt_best_ns", ctypes.c_double),
        ("worst_sender_xcc", ctypes.c_int),
        ("worst_receiver_xcc", ctypes.c_int),
        ("pairs", ctypes.c_int),
    ]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m latency_collectives_amd.build`")
    # torch bundles its own HIP runtime with the same soname as /opt/rocm's. Loading torch first
    # makes libar.so bind to that one runtime, so torch's streams and allocations are valid in
    # the library (two runtimes in one process would not share devices or streams).
    import torch  # noqa: F401

    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64, u64 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64,
                             ctypes.c_uint64)
    pp = ctypes.POINTER(ctypes.c_void_p)
    pu64 = ctypes.POINTER(ctypes.c_uint64)
    pdbl = ctypes.POINTER(ctypes.c_double)
    sig = {
        "ar_create": ([i32, sz, i32], vp),
        "ar_allreduce": ([vp, pp, pp, sz, i32, vp], i32),
        "ar_allreduce_noalloc": ([i32, i32, pp, pp, sz, i32, vp], i32),
        "ar_reducescatter": ([vp, pp, pp, sz, vp], i32),
        "ar_allgather": ([vp, pp, pp, sz, vp], i32),
        "ar_broadcast": ([vp, vp, pp, sz, i32, vp], i32),
        "ar_destroy": ([vp], None),
        "ar_last_error": ([], ctypes.c_char_p),
        "ar_check": ([vp], i32),
        "ar_bench": ([vp, pp, pp, i32, sz, i32, i32, pu64, pu64, vp], i32),
        "ar_bench_ex": ([vp, pp, pp, i32, sz, i32, i32, pu64, pu64, pdbl, vp], i32),
        "ar_wallclock_hz": ([], ctypes.c_double),
        "ar_set_option": ([vp, i32, i64], i32),
        "ar_region_bytes": ([vp, i32], i64),
        "ar_alg_bytes": ([vp, sz, i32], i64),
        "ar_plan_info": ([vp, sz, i32, ctypes.POINTER(ar_plan)], i32),
        "ar_read_region": ([vp, i32, i32, vp, sz], i32),
        "ar_epoch": ([vp], u64),
        "ar_sol": ([i32, pdbl], i32),
        "ar_sol_ex": ([i32, ctypes.POINTER(ar_sol_result)], i32),
        "ar_sol_ranks": ([i32, i32, ctypes.POINTER(ar_sol_ranks_result)], i32),
        "ar_pingpong": ([i32, i32, i32, i32, pdbl, ctypes.POINTER(ctypes.c_int)], i32),
        "ar_torn_lines": ([i32, i32, i32, pu64, pu64], i32),
        "ar_stream_copy": ([vp, vp, sz, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def ar_last_error() -> str:
    return lib().ar_last_error().decode(errors="replace")


def _ok(rc: int) -> int:
    if rc != AR_OK:
        raise ArError(rc, ar_last_error())
    return rc


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> int:
    if s is None:
        import torch

        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _table(ptrs):
    tab = (ctypes.c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        tab[i] = _ptr(p)
    return tab


def ar_create(nranks: int, max_bytes: int, dtype: int) -> int:
    h = lib().ar_create(int(nranks), int(max_bytes), int(dtype))
    if not h:
        raise ArError(AR_EINVAL, ar_last_error())
    return int(h)


def ar_destroy(h: int) -> None:
    lib().ar_destroy(h)


def ar_allreduce(h: int, ins, outs, count: int, algo: int, stream=None) -> None:
    _ok(lib().ar_allreduce(h, _table(ins), _table(outs), int(count), int(algo), _stream(stream)))


def ar_allreduce_noalloc(nranks: int, dtype: int, ins, outs, count: int, algo: int,
                         stream=None) -> None:
    _ok(lib().ar_allreduce_noalloc(int(nranks), int(dtype), _table(ins), _table(outs),
                                   int(count), int(algo), _stream(stream)))


def ar_reducescatter(h: int, ins, outs, recvcount: int, stream=None) -> None:
    _ok(lib().ar_reducescatter(h, _table(ins), _table(outs), int(recvcount), _stream(stream)))


def ar_allgather(h: int, ins, outs, sendcount: int, stream=None) -> None:
    _ok(lib().ar_allgather(h, _table(ins), _table(outs), int(sendcount), _stream(stream)))


def ar_broadcast(h: int, inp, outs, count: int, root: int, stream=None) -> None:
    _ok(lib().ar_broadcast(h, _ptr(inp), _table(outs), int(count), int(root), _stream(stream)))


def ar_check(h: int) -> None:
    _ok(lib().ar_check(h))


def _bench_args(in_sets, out_sets, nsets: int, iters: int, timestamps: bool):
    import numpy as np

    n = len(in_sets) // max(nsets, 1) if in_sets else 0
    ts = te = None
    p_ts = p_te = None
    if timestamps and n:
        ts = np.zeros(iters * n, dtype=np.uint64)
        te = np.zeros(iters * n, dtype=np.uint64)
        p_ts = ts.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
        p_te = te.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    tin = _table(in_sets) if in_sets else None
    tout = _table(out_sets) if out_sets else None
    return ts, te, p_ts, p_te, tin, tout


def ar_bench(h: int, in_sets, out_sets, nsets: int, count: int, algo: int, iters: int,
             timestamps: bool = True, stream=None):
    """Returns (t_start, t_end): arrays of iters * N ticks, or None without timestamps."""
    ts, te, p_ts, p_te, tin, tout = _bench_args(in_sets, out_sets, nsets, iters, timestamps)
    _ok(lib().ar_bench(h, tin, tout, int(nsets), int(count), int(algo), int(iters), p_ts, p_te,
                       _stream(stream)))
    return ts, te


def ar_bench_ex(h: int, in_sets, out_sets, nsets: int, count: int, algo: int, iters: int,
                timestamps: bool = True, stream=None):
    """Returns (t_start, t_end, elapsed_ms)."""
    ts, te, p_ts, p_te, tin, tout = _bench_args(in_sets, out_sets, nsets, iters, timestamps)
    ms = ctypes.c_double(0.0)
    _ok(lib().ar_bench_ex(h, tin, tout, int(nsets), int(count), int(algo), int(iters), p_ts,
                          p_te, ctypes.byref(ms), _stream(stream)))
    return ts, te, ms.value


def ar_wallclock_hz() -> float:
    return float(lib().ar_wallclock_hz())


def ar_set_option(h: int, opt: int, value: int) -> None:
    _ok(lib().ar_set_option(h, int(opt), int(value)))


def ar_alg_bytes(h: int, count: int, algo: int) -> int:
    v = int(lib().ar_alg_bytes(h, int(count), int(algo)))
    if v < 0:
        raise ArError(v, ar_last_error())
    return v


def ar_plan_info(h: int, count: int, algo: int) -> dict:
    p = ar_plan()
    _ok(lib().ar_plan_info(h, int(count), int(algo), ctypes.byref(p)))
    return p.as_dict()


def ar_region_bytes(h: int, region: int) -> int:
    v = int(lib().ar_region_bytes(h, int(region)))
    if v < 0:
        raise ArError(v, ar_last_error())
    return v


def ar_read_region(h: int, rank: int, region: int, nbytes: int | None = None):
    import numpy as np

    if nbytes is None:
        nbytes = ar_region_bytes(h, region)
    buf = np.empty(nbytes, dtype=np.uint8)
    _ok(lib().ar_read_region(h, int(rank), int(region), buf.ctypes.data, int(nbytes)))
    return buf


def ar_epoch(h: int) -> int:
    return int(lib().ar_epoch(h))


def ar_sol(placement: int = AR_PLACE_XCD) -> dict:
    """{fence_ns, l2_load_ns, store_half_rtt_ns} (the three terms of the pages' bound)."""
    out = (ctypes.c_double * 3)()
    _ok(lib().ar_sol(int(placement), out))
    return {"fence_ns": out[0], "l2_load_ns": out[1], "store_half_rtt_ns": out[2]}


def ar_sol_ex(placement: int = AR_PLACE_XCD) -> dict:
    res = ar_sol_result()
    _ok(lib().ar_sol_ex(int(placement), ctypes.byref(res)))
    return res.as_dict()


def ar_sol_ranks(nranks: int, placement: int = AR_PLACE_XCD) -> dict:
    res = ar_sol_ranks_result()
    _ok(lib().ar_sol_ranks(int(nranks), int(placement), ctypes.byref(res)))
    return res.as_dict()


def ar_pingpong(placement: int, store_policy: int, load_policy: int, rounds: int):
    half = ctypes.c_double(0.0)
    xcc = (ctypes.c_int * 2)(-1, -1)
    _ok(lib().ar_pingpong(int(placement), int(store_policy), int(load_policy), int(rounds),
                          ctypes.byref(half), xcc))
    return half.value, (xcc[0], xcc[1])


def ar_torn_lines(placement: int, nlines: int, gens: int):
    torn = ctypes.c_uint64(0)
    reads = ctypes.c_uint64(0)
    _ok(lib().ar_torn_lines(int(placement), int(nlines), int(gens), ctypes.byref(torn),
                            ctypes.byref(reads)))
    return torn.value, reads.value


def ar_stream_copy(dst, src, nbytes: int, stream=None) -> None:
    _ok(lib().ar_stream_copy(_ptr(dst), _ptr(src), int(nbytes), _stream(stream)))
