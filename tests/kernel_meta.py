"""The gfx950 code objects of latency_collectives_amd/libar.so, read with the ROCm LLVM tools
(no GPU needed): each kernel's disassembly and its code-object metadata (register counts,
LDS and private segment sizes), and the number of its workgroups one compute unit can hold,
computed from that metadata alone.

Occupancy of a gfx950 compute unit (CDNA: 4 SIMDs of 64-lane waves; a compute unit holds
4 x (waves per SIMD) waves, a workgroup of W waves takes W of them):
  - VGPRs: 512 per lane per SIMD, shared by the architectural and accumulation registers
    (the metadata's vgpr_count is their unified total), allocated in blocks of 8;
  - SGPRs: the gfx9 rule (at most 10 waves per SIMD up to 80 SGPRs, 9 up to 88, 8 up to 100,
    7 beyond);
  - wave slots: `max_waves_per_simd` (8 on CDNA3/4: 2048 threads per compute unit);
  - LDS: 160 KiB per compute unit.
A kernel with a private segment (register spills, a stack) also needs scratch that the runtime
backs for a limited number of waves, which this count does not see; the product's kernels have
none (checked on the CPU)."""

from __future__ import annotations

import os
import re
import shutil
import struct
import subprocess

import yaml

LLVM = "/opt/rocm/llvm/bin"
VGPRS_PER_SIMD = 512
VGPR_GRANULE = 8
SIMDS_PER_CU = 4
LDS_PER_CU = 160 * 1024


def tools_available() -> bool:
    return (os.path.exists(os.path.join(LLVM, "clang-offload-bundler"))
            and os.path.exists(os.path.join(LLVM, "llvm-objdump"))
            and os.path.exists(os.path.join(LLVM, "llvm-readelf"))
            and shutil.which("objcopy") is not None)


def code_objects(lib: str, workdir: str) -> list:
    """Unbundle every translation unit's gfx950 code object out of `lib` into `workdir`."""
    fat = os.path.join(workdir, "fat.bin")
    subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", lib], check=True)
    # one offload bundle per translation unit, concatenated (each starts with the magic string)
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    raw = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(magic), raw)]
    out = []
    for j, a in enumerate(starts):
        part, co = os.path.join(workdir, f"fat{j}.bin"), os.path.join(workdir, f"co{j}.o")
        with open(part, "wb") as f:
            f.write(raw[a:starts[j + 1] if j + 1 < len(starts) else len(raw)])
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        f"--input={part}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--output={co}"], check=True)
        out.append(co)
    return out


def disassembly(objs: list) -> dict:
    """Kernel symbol -> its instructions (text, one per line)."""
    text = "".join(subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                                  check=True, capture_output=True, text=True).stdout
                   for co in objs)
    out, name = {}, None
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            name = m.group(1)
            out[name] = []
        elif name is not None and line.startswith("\t"):
            out[name].append(line.strip())
    return out


def _sections(elf: bytes) -> dict:
    """Section name -> (type, file offset, size) of a little-endian ELF64 image."""
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    hdr = [struct.unpack_from("<IIQQQQIIQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    strtab = hdr[shstrndx][4]
    out = {}
    for h in hdr:
        name = elf[strtab + h[0]:elf.index(b"\0", strtab + h[0])].decode()
        out.setdefault(name, (h[1], h[4], h[5]))
        if h[1] == 7:  # SHT_NOTE: keep every note section
            out.setdefault("notes", [])
            out["notes"].append((h[4], h[5]))
    return out


def metadata_from_library(lib: str) -> dict:
    """Kernel symbol -> its amdhsa.kernels metadata record, read from `lib` in plain Python (no
    tool is started: a process that uses the GPU should not fork and exec): the .hip_fatbin
    section holds one offload bundle per translation unit, each bundle its gfx950 code object,
    and each code object an NT_AMDGPU_METADATA note (MessagePack)."""
    import msgpack

    raw = open(lib, "rb").read()
    _, off, size = _sections(raw)[".hip_fatbin"]
    fat = raw[off:off + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    out = {}
    for m in re.finditer(re.escape(magic), fat):
        b = m.start()
        (n,) = struct.unpack_from("<Q", fat, b + len(magic))
        p = b + len(magic) + 8
        for _ in range(n):
            eoff, esize, tlen = struct.unpack_from("<QQQ", fat, p)
            triple = fat[p + 24:p + 24 + tlen].decode()
            p += 24 + tlen
            if not triple.endswith("gfx950"):
                continue
            co = fat[b + eoff:b + eoff + esize]
            for noff, nsize in _sections(co).get("notes", []):
                q = noff
                while q < noff + nsize:
                    namesz, descsz, ntype = struct.unpack_from("<III", co, q)
                    name = co[q + 12:q + 12 + namesz].rstrip(b"\0")
                    d0 = q + 12 + (namesz + 3) // 4 * 4
                    if ntype == 32 and name == b"AMDGPU":
                        doc = msgpack.unpackb(co[d0:d0 + descsz], raw=False)
                        for k in doc.get("amdhsa.kernels") or []:
                            out[k[".symbol"].removesuffix(".kd")] = k
                    q = d0 + (descsz + 3) // 4 * 4
    return out


def metadata(objs: list) -> dict:
    """Kernel symbol -> its amdhsa.kernels metadata record, read with llvm-readelf."""
    out = {}
    for co in objs:
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co], check=True,
                               capture_output=True, text=True).stdout
        doc = yaml.safe_load(notes[notes.index("---"):notes.rindex("...")])
        for k in doc.get("amdhsa.kernels") or []:
            out[k[".symbol"].removesuffix(".kd")] = k
    return out


def waves_per_simd(meta: dict, max_waves_per_simd: int = 8, sgpr_rule: bool = True) -> int:
    v = -(-max(1, int(meta[".vgpr_count"])) // VGPR_GRANULE) * VGPR_GRANULE
    by_vgpr = VGPRS_PER_SIMD // v
    s = int(meta[".sgpr_count"])
    by_sgpr = (10 if s <= 80 else 9 if s <= 88 else 8 if s <= 100 else 7) if sgpr_rule else 99
    return min(by_vgpr, by_sgpr, max_waves_per_simd)


def workgroups_per_cu(meta: dict, threads: int, max_waves_per_simd: int = 8,
                      sgpr_rule: bool = True) -> int:
    """Workgroups of `threads` threads of this kernel that one compute unit holds at once
    (`sgpr_rule` False: the VGPR, wave-slot and LDS limits only, an upper bound)."""
    waves = -(-threads // 64)
    by_regs = SIMDS_PER_CU * waves_per_simd(meta, max_waves_per_simd, sgpr_rule) // waves
    lds = int(meta[".group_segment_fixed_size"])
    by_lds = LDS_PER_CU // lds if lds else by_regs
    return min(by_regs, by_lds)


def kernel_symbol(kernel: int, dt: int, nmax: int) -> str:
    """Mangled name of the AllReduce kernel of family `kernel` (7: the bulk two-shot) for dtype
    id `dt` (0 fp32, 1 bf16, 2 int32) and rank bound `nmax`."""
    if kernel == 7:
        return f"_ZN2ar14ar_kernel_bulkILi{dt}ELi{nmax}EEEvNS_4ArgsE"
    return f"_ZN2ar9ar_kernelILi{kernel}ELi{dt}ELi{nmax}EEEvNS_4ArgsE"
