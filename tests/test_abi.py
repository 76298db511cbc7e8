"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, and
rejects bad arguments before touching the device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def arlib():
    from latency_collectives_amd import build

    build.ensure_built()
    from latency_collectives_amd import _ar

    return _ar


def _declared():
    with open(os.path.join(ROOT, "include", "ar.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("ar_create", "ar_allreduce", "ar_destroy"):
        assert must in names


def test_every_declared_symbol_is_exported(arlib):
    L = arlib.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert sorted(arlib.EXPORTS) == _declared()


def test_create_rejects_bad_arguments(arlib):
    L = arlib.lib()
    assert not L.ar_create(0, 1024, 0)
    assert "nranks" in arlib.ar_last_error()
    assert not L.ar_create(17, 1024, 0)
    assert not L.ar_create(2, 0, 0)
    assert "max_bytes" in arlib.ar_last_error()
    assert not L.ar_create(2, 1 << 31, 0)
    assert not L.ar_create(2, 1024, 7)
    assert "dtype" in arlib.ar_last_error()


def test_null_handle_calls_fail_cleanly(arlib):
    L = arlib.lib()
    assert L.ar_allreduce(None, None, None, 0, 0, None) == arlib.AR_EINVAL
    assert L.ar_check(None) == arlib.AR_EINVAL
    assert L.ar_set_option(None, 0, 1) == arlib.AR_EINVAL
    assert L.ar_bench(None, None, None, 1, 1, 1, 1, None, None, None) == arlib.AR_EINVAL
    assert L.ar_bench_ex(None, None, None, 1, 1, 1, 1, None, None, None, None) == arlib.AR_EINVAL
    assert L.ar_region_bytes(None, 0) == arlib.AR_EINVAL
    assert L.ar_epoch(None) == 0
    assert L.ar_reducescatter(None, None, None, 4, None) == arlib.AR_EINVAL
    assert L.ar_allgather(None, None, None, 4, None) == arlib.AR_EINVAL
    assert L.ar_broadcast(None, None, None, 4, 0, None) == arlib.AR_EINVAL
    assert L.ar_alg_bytes(None, 4, 1) == arlib.AR_EINVAL
    assert L.ar_plan_info(None, 4, 1, None) == arlib.AR_EINVAL
    L.ar_destroy(None)  # must be a no-op


def test_sol_and_probe_argument_checks(arlib):
    L = arlib.lib()
    assert L.ar_sol(0, None) == arlib.AR_EINVAL
    assert L.ar_sol_ex(0, None) == arlib.AR_EINVAL
    assert L.ar_sol_ranks(4, 0, None) == arlib.AR_EINVAL
    assert L.ar_stream_copy(None, None, 16, None) == arlib.AR_EINVAL
    half = ctypes.c_double()
    assert L.ar_pingpong(0, 3, 16, 10, ctypes.byref(half), None) == arlib.AR_EINVAL
    t = ctypes.c_uint64()
    assert L.ar_torn_lines(0, 0, 10, ctypes.byref(t), ctypes.byref(t)) == arlib.AR_EINVAL


def test_binding_names_match_c_entry_points(arlib):
    for name in arlib.EXPORTS:
        assert callable(getattr(arlib, name)), name


def test_binding_constants_match_the_header(arlib):
    """Every AR_* constant the header defines with an explicit value (data types, algorithms,
    error codes, placements, options) has the same value in the Python binding."""
    with open(os.path.join(ROOT, "include", "ar.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    consts = dict((k, int(v)) for k, v in re.findall(r"\b(AR_[A-Z0-9_]+)\s*=\s*(-?\d+)", text))
    assert len(consts) > 30
    missing = [k for k in consts if not hasattr(arlib, k)]
    assert not missing, missing
    wrong = {k: (v, getattr(arlib, k)) for k, v in consts.items() if getattr(arlib, k) != v}
    assert not wrong, wrong
