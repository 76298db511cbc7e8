"""Checks on the gfx950 machine code this repository builds (no GPU needed): the code object is
taken out of latency_collectives_amd/libar.so and disassembled with the ROCm LLVM tools.

They pin the properties the design relies on: LL lines and sentinel slots move as single
16-byte vector accesses (8-byte ones in the narrow kernels), cross-rank accesses carry the
agent-coherent policy and the bulk kernel's input and output streams the non-temporal one, and
no packed fp32 arithmetic appears anywhere (the build disables it)."""

import os
import re
import shutil
import subprocess

import pytest

LLVM = "/opt/rocm/llvm/bin"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    from latency_collectives_amd import build

    lib = build.ensure_built()
    bundler = os.path.join(LLVM, "clang-offload-bundler")
    objdump = os.path.join(LLVM, "llvm-objdump")
    if not (os.path.exists(bundler) and os.path.exists(objdump) and shutil.which("objcopy")):
        pytest.skip("ROCm LLVM tools or objcopy not available")
    d = tmp_path_factory.mktemp("isa")
    fat = str(d / "fat.bin")
    subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", lib], check=True)
    # one offload bundle per translation unit, concatenated (each starts with the magic string)
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    raw = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(magic), raw)]
    text = ""
    for j, a in enumerate(starts):
        part, co = str(d / f"fat{j}.bin"), str(d / f"co{j}.o")
        with open(part, "wb") as f:
            f.write(raw[a:starts[j + 1] if j + 1 < len(starts) else len(raw)])
        subprocess.run([bundler, "--unbundle", "--type=o", f"--input={part}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                       check=True)
        text += subprocess.run([objdump, "-d", "--mcpu=gfx950", co], check=True,
                               capture_output=True, text=True).stdout
    out, name = {}, None
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            name = m.group(1)
            out[name] = []
        elif name is not None and line.startswith("\t"):
            out[name].append(line.strip())
    return out


def _kernel(kernels, algo, dt, nmax, bulk=False):
    sym = (f"_ZN2ar14ar_kernel_bulkILi{dt}ELi{nmax}EEEvNS_4ArgsE" if bulk
           else f"_ZN2ar9ar_kernelILi{algo}ELi{dt}ELi{nmax}EEEvNS_4ArgsE")
    assert sym in kernels, sym
    return kernels[sym]


def _ops(ins, op):
    return [i for i in ins if i.split()[0] == op]


def test_ll_lines_are_single_16_byte_accesses(kernels):
    """One-shot LL, fp32, N = 2: pushes and polls are 16-byte buffer accesses with the
    agent-coherent policy ({8 bytes payload, 8 bytes sequence number} in one store)."""
    ins = _kernel(kernels, 1, 0, 2)
    st = [i for i in _ops(ins, "buffer_store_dwordx4") if "sc1" in i]
    ld = [i for i in _ops(ins, "buffer_load_dwordx4") if "sc1" in i]
    assert st and ld


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
