"""Python access to the CPU oracle (TEST INFRASTRUCTURE ONLY).

The oracle is the plain C++ AllReduce in ``allreduce_ref.cpp`` (left fold over ranks 0..N-1,
binary32 accumulation, one round-to-nearest-even for bfloat16, wrapping int32; see the header of
that file for the passages it follows). This module builds it with g++ and calls it through
ctypes on numpy arrays. Only the tests, the smoke check and the benchmark's CPU-baseline leg
import this module; the product path never does.

bfloat16 data is carried as ``numpy.uint16`` bit patterns (numpy has no bfloat16 dtype).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "allreduce_ref.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

# No fast-math and no floating-point contraction: the fold must round after every addition.
_CFLAGS = ["-O2", "-std=c++17", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]

_lib = None


def build(force: bool = True) -> str:
    """Compile ``allreduce_ref.cpp`` into ``liboracle.so`` next to it and return the path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["g++", *_CFLAGS, _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    """Load the oracle library, building it first only if no built copy exists."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        pp = ctypes.POINTER(ctypes.c_void_p)
        for name in ("oracle_allreduce_f32", "oracle_allreduce_f64", "oracle_allreduce_bf16",
                     "oracle_allreduce_i32"):
            fn = getattr(L, name)
            fn.argtypes = [ctypes.c_int, pp, pp, ctypes.c_size_t]
            fn.restype = ctypes.c_int
        for name in ("oracle_reducescatter_f32", "oracle_reducescatter_f64",
                     "oracle_reducescatter_bf16", "oracle_reducescatter_i32", "oracle_allgather"):
            fn = getattr(L, name)
            fn.argtypes = [ctypes.c_int, pp, pp, ctypes.c_size_t]
            fn.restype = ctypes.c_int
        for name in ("oracle_allreduce_grouped_f32", "oracle_allreduce_grouped_bf16"):
            fn = getattr(L, name)
            fn.argtypes = [ctypes.c_int, ctypes.c_int, pp, pp, ctypes.c_size_t]
            fn.restype = ctypes.c_int
        L.oracle_broadcast.argtypes = [ctypes.c_int, ctypes.c_void_p, pp, ctypes.c_size_t]
        L.oracle_broadcast.restype = ctypes.c_int
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_time_allreduce.argtypes = [ctypes.c_int, ctypes.c_int, pp, pp, ctypes.c_size_t,
                                            ctypes.c_int]
        L.oracle_time_allreduce.restype = ctypes.c_double
        _lib = L
    return _lib


_FN = {
    np.dtype(np.float32): "oracle_allreduce_f32",
    np.dtype(np.float64): "oracle_allreduce_f64",
    np.dtype(np.uint16): "oracle_allreduce_bf16",
    np.dtype(np.int32): "oracle_allreduce_i32",
}
_TIME_CODE = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.int32): 2}


def _ptr_table(arrays):
    tab = (ctypes.c_void_p * len(arrays))()
    for i, a in enumerate(arrays):
        tab[i] = a.ctypes.data
    return tab


def _check(arrays):
    if len(arrays) < 1:
        raise ValueError("need at least one rank")
    dt = arrays[0].dtype
    n = arrays[0].size
    for a in arrays:
        if a.dtype != dt or a.size != n or a.ndim != 1 or not a.flags.c_contiguous:
            raise ValueError("all ranks need 1-D contiguous arrays of one dtype and size")
    if dt not in _FN:
        raise TypeError(f"unsupported dtype {dt}")
    return dt, n


def allreduce(arrays, out=None):
    """AllReduce-sum of ``arrays`` (one 1-D array per rank). Returns one output array per rank.

    ``out`` may be given (a list of arrays like ``arrays``); an output may be the matching input.
    """
    dt, n = _check(arrays)
    if out is None:
        out = [np.empty(n, dtype=dt) for _ in arrays]
    _check(out)
    fn = getattr(lib(), _FN[dt])
    rc = fn(len(arrays), _ptr_table(arrays), _ptr_table(out), n)
    if rc != 0:
        raise ValueError(f"oracle rejected arguments (rc={rc})")
    return out


_GROUPED_FN = {
    np.dtype(np.float32): "oracle_allreduce_grouped_f32",
    np.dtype(np.uint16): "oracle_allreduce_grouped_bf16",
}


def allreduce_grouped(arrays, group: int):
    """AllReduce-sum in the hierarchical order of the deterministic atomic variant: groups of
    ``group`` consecutive ranks are folded in rank order, then the group sums in group order
    (binary32; bfloat16 rounded once). fp32 and bf16 only (an int32 sum does not depend on the
    order). Returns one output array per rank."""
    dt, n = _check(arrays)
    if dt not in _GROUPED_FN:
        raise TypeError(f"no grouped fold for {dt}")
    out = [np.empty(n, dtype=dt) for _ in arrays]
    rc = getattr(lib(), _GROUPED_FN[dt])(len(arrays), int(group), _ptr_table(arrays),
                                         _ptr_table(out), n)
    if rc != 0:
        raise ValueError(f"oracle rejected arguments (rc={rc})")
    return out


_RS_FN = {
    np.dtype(np.float32): "oracle_reducescatter_f32",
    np.dtype(np.float64): "oracle_reducescatter_f64",
    np.dtype(np.uint16): "oracle_reducescatter_bf16",
    np.dtype(np.int32): "oracle_reducescatter_i32",
}


def reducescatter(arrays):
    """Reduce-scatter-sum: ``arrays`` holds one 1-D input per rank, N partitions of
    ``size // N`` elements each; returns rank r's output (the fold of partition r over ranks)."""
    dt, n = _check(arrays)
    N = len(arrays)
    if n % N != 0:
        raise ValueError("input length must be a multiple of the rank count")
    rc_n = n // N
    out = [np.empty(rc_n, dtype=dt) for _ in arrays]
    rc = getattr(lib(), _RS_FN[dt])(N, _ptr_table(arrays), _ptr_table(out), rc_n)
    if rc != 0:
        raise ValueError(f"oracle rejected arguments (rc={rc})")
    return out


def allgather(arrays):
    """All-gather: returns, per rank, the concatenation of every rank's input in rank order."""
    dt, n = _check(arrays)
    N = len(arrays)
    out = [np.empty(N * n, dtype=dt) for _ in arrays]
    rc = lib().oracle_allgather(N, _ptr_table(arrays), _ptr_table(out), n * dt.itemsize)
    if rc != 0:
        raise ValueError(f"oracle rejected arguments (rc={rc})")
    return out


def broadcast(root_in: np.ndarray, nranks: int):
    """Broadcast: returns ``nranks`` outputs, each a copy of ``root_in``."""
    root_in = np.ascontiguousarray(root_in)
    out = [np.empty_like(root_in) for _ in range(nranks)]
    rc = lib().oracle_broadcast(int(nranks), root_in.ctypes.data, _ptr_table(out),
                                root_in.nbytes)
    if rc != 0:
        raise ValueError(f"oracle rejected arguments (rc={rc})")
    return out


def allreduce_rows(x: np.ndarray) -> np.ndarray:
    """Convenience form: ``x`` has shape [N, count]; returns the single reduced row."""
    x = np.ascontiguousarray(x)
    rows = [x[r] for r in range(x.shape[0])]
    return allreduce(rows)[0]


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns (round to nearest even), element by element."""
    L = lib()
    flat = np.asarray(x, dtype=np.float32).ravel()
    return np.array([L.oracle_f32_to_bf16(float(v)) for v in flat], dtype=np.uint16).reshape(
        np.shape(x))


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> binary32 (exact), element by element."""
    L = lib()
    flat = np.asarray(b, dtype=np.uint16).ravel()
    return np.array([L.oracle_bf16_to_f32(int(v)) for v in flat], dtype=np.float32).reshape(
        np.shape(b))


def time_allreduce(arrays, reps: int) -> float:
    """Seconds for ``reps`` single-threaded oracle AllReduces over ``arrays`` (host memory)."""
    dt, n = _check(arrays)
    if dt not in _TIME_CODE:
        raise TypeError(f"no timing entry for {dt}")
    out = [np.empty(n, dtype=dt) for _ in arrays]
    s = lib().oracle_time_allreduce(_TIME_CODE[dt], len(arrays), _ptr_table(arrays),
                                    _ptr_table(out), n, int(reps))
    if s < 0:
        raise ValueError("oracle timing rejected arguments")
    return float(s)
