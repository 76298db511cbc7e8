"""Checks on the gfx950 machine code this repository builds (no GPU needed): the code object is
taken out of latency_collectives_amd/libar.so and disassembled with the ROCm LLVM tools.

They pin the properties the design relies on: LL lines and sentinel slots move as single
16-byte vector accesses (8-byte ones in the narrow kernels), cross-rank accesses carry the
agent-coherent policy and the bulk kernel's input and output streams the non-temporal one, and
no packed fp32 arithmetic appears anywhere (the build disables it)."""

import re

import pytest

from tests import kernel_meta as KM


@pytest.fixture(scope="module")
def objs(tmp_path_factory):
    from latency_collectives_amd import build

    lib = build.ensure_built()
    if not KM.tools_available():
        pytest.skip("ROCm LLVM tools or objcopy not available")
    return KM.code_objects(lib, str(tmp_path_factory.mktemp("isa")))


@pytest.fixture(scope="module")
def kernels(objs):
    return KM.disassembly(objs)


@pytest.fixture(scope="module")
def meta(objs):
    return KM.metadata(objs)


def _kernel(kernels, algo, dt, nmax, bulk=False):
    sym = (f"_ZN2ar14ar_kernel_bulkILi{dt}ELi{nmax}EEEvNS_4ArgsE" if bulk
           else f"_ZN2ar9ar_kernelILi{algo}ELi{dt}ELi{nmax}EEEvNS_4ArgsE")
    assert sym in kernels, sym
    return kernels[sym]


def _ops(ins, op):
    return [i for i in ins if i.split()[0] == op]


def test_ll_lines_are_single_16_byte_accesses(kernels):
    """One-shot LL, fp32, N = 2, and the peer-split LL kernel, N = 16: pushes and polls are
    16-byte buffer accesses with the agent-coherent policy ({8 bytes payload, 8 bytes sequence
    number} in one store)."""
    for fam, nmax in ((1, 2), (33, 16)):
        ins = _kernel(kernels, fam, 0, nmax)
        st = [i for i in _ops(ins, "buffer_store_dwordx4") if "sc1" in i]
        ld = [i for i in _ops(ins, "buffer_load_dwordx4") if "sc1" in i]
        assert st and ld, fam


def test_sentinel_kernels_unit_widths(kernels):
    """One-shot sentinel, bf16, N = 4: the 16-byte kernel pushes and polls dwordx4, the
    narrow kernel dwordx2, both coherent."""
    wide = _kernel(kernels, 2, 1, 4)
    narrow = _kernel(kernels, 10, 1, 4)
    assert [i for i in _ops(wide, "buffer_store_dwordx4") if "sc1" in i]
    assert [i for i in _ops(wide, "buffer_load_dwordx4") if "sc1" in i]
    assert [i for i in _ops(narrow, "buffer_store_dwordx2") if "sc1" in i]
    assert [i for i in _ops(narrow, "buffer_load_dwordx2") if "sc1" in i]


def test_bulk_two_shot_cache_policies(kernels):
    """Bulk two-shot, int32, N = 8: input loads non-temporal, pushes and slot reads coherent,
    all 16 bytes wide."""
    ins = _kernel(kernels, 0, 2, 8, bulk=True)
    loads = _ops(ins, "buffer_load_dwordx4")
    stores = _ops(ins, "buffer_store_dwordx4")
    assert [i for i in loads if re.search(r"\bnt\b", i)]
    assert [i for i in loads if "sc1" in i]
    assert [i for i in stores if "sc1" in i]
    assert [i for i in stores if re.search(r"\bnt\b", i)]


def test_no_packed_fp32_arithmetic(kernels):
    bad = [(k, i) for k, ins in kernels.items() for i in ins
           if i.split()[0] in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")]
    assert not bad, bad[:4]


def test_no_kernel_has_a_private_segment(meta):
    """Every wave of an AllReduce grid polls for the others, so the whole grid must be resident
    at once, and the planner counts residency from registers and LDS (the occupancy query). A
    kernel that spills to the private segment also needs scratch, which the runtime may back for
    fewer waves than the registers allow: no kernel of the library has a private segment or a
    dynamic stack."""
    assert meta
    bad = {k: (m[".private_segment_fixed_size"], m[".vgpr_spill_count"])
           for k, m in meta.items()
           if m[".private_segment_fixed_size"] or m[".uses_dynamic_stack"]}
    assert not bad, bad


def test_every_allreduce_kernel_fits_the_planner_shapes(meta):
    """The planner launches 64..256 threads per workgroup and at least one workgroup per compute
    unit: every AllReduce kernel accepts 256-thread workgroups and one compute unit holds at
    least one of them, with 64-lane waves; the bulk two-shot kernels for up to 8 ranks hold at
    least two (the planner keeps one free; with 16 ranks and bf16 the register budget gives one
    workgroup per compute unit)."""
    ar = {k: m for k, m in meta.items() if k.startswith(("_ZN2ar9ar_kernel", "_ZN2ar14ar_kernel"))}
    assert len(ar) > 100
    for k, m in ar.items():
        assert m[".wavefront_size"] == 64, k
        assert m[".max_flat_workgroup_size"] >= 256, k
        assert KM.workgroups_per_cu(m, 256) >= 1, k
        if "bulk" in k and not k.endswith("ELi16EEEvNS_4ArgsE"):
            assert KM.workgroups_per_cu(m, 256) >= 2, (k, m[".vgpr_count"])


def test_metadata_reader_agrees_with_llvm_readelf(meta):
    """The plain-Python reader of the code-object metadata (used by GPU tests, which must not
    start tools from a process that uses the GPU) gives llvm-readelf's records."""
    from latency_collectives_amd import build

    mine = KM.metadata_from_library(build.ensure_built())
    assert set(mine) == set(meta)
    keys = (".vgpr_count", ".agpr_count", ".sgpr_count", ".group_segment_fixed_size",
            ".private_segment_fixed_size", ".max_flat_workgroup_size", ".wavefront_size")
    for k, m in meta.items():
        assert [mine[k][x] for x in keys] == [m[x] for x in keys], k
