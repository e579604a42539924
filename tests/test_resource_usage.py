"""Register and scratch usage of every kernel in the built library.

Each kernel runs one wave per SIMD and keeps its in-flight K/V chunks in
registers.  A kernel that needs more vector registers than gfx950 gives a
wave spills some of them (into accumulation registers, or into scratch
memory); a spilled register that is the destination of a load still in
flight has given wrong results.  So no kernel may spill vector registers or
use scratch memory.  The check reads the AMDGPU metadata note of the gfx950
code object inside libpagedkv.so: no GPU is needed.
"""
import os
import struct

import pytest

msgpack = pytest.importorskip("msgpack")

import paged_kv_cache_100_amd as pkv

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NT_AMDGPU_METADATA = 32


def _sections(elf: bytes):
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    heads = [struct.unpack_from("<IIQQQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    strtab_off = heads[shstrndx][4]

    def name(n):
        end = elf.index(b"\0", strtab_off + n)
        return elf[strtab_off + n:end].decode()

    return {name(h[0]): (h[1], h[4], h[5]) for h in heads}


def _gfx950_code_object(lib: bytes) -> bytes:
    typ, off, size = _sections(lib)[".hip_fatbin"]
    fat = lib[off:off + size]
    assert fat.startswith(BUNDLE_MAGIC), "offload bundle not found (compressed bundle?)"
    pos = len(BUNDLE_MAGIC)
    (count,) = struct.unpack_from("<Q", fat, pos)
    pos += 8
    for _ in range(count):
        e_off, e_size, id_len = struct.unpack_from("<QQQ", fat, pos)
        pos += 24
        ident = fat[pos:pos + id_len].decode()
        pos += id_len
        if ident.startswith("hip") and ident.endswith("gfx950"):
            return fat[e_off:e_off + e_size]
    raise AssertionError("no gfx950 code object in the library")


def _metadata(code: bytes) -> dict:
    for typ, off, size in _sections(code).values():
        if typ != 7:                                   # SHT_NOTE
            continue
        pos, end = off, off + size
        while pos + 12 <= end:
            namesz, descsz, ntype = struct.unpack_from("<III", code, pos)
            name = code[pos + 12:pos + 12 + namesz].rstrip(b"\0")
            desc_off = pos + 12 + (namesz + 3) // 4 * 4
            if ntype == NT_AMDGPU_METADATA and name == b"AMDGPU":
                return msgpack.unpackb(code[desc_off:desc_off + descsz], raw=False)
            pos = desc_off + (descsz + 3) // 4 * 4
    raise AssertionError("no AMDGPU metadata note in the code object")


@pytest.fixture(scope="module")
def kernels():
    path = pkv.LIB_PATH
    if not os.path.exists(path):
        pytest.skip("libpagedkv.so is not built")
    with open(path, "rb") as f:
        meta = _metadata(_gfx950_code_object(f.read()))
    ks = meta["amdhsa.kernels"]
    assert ks, "no kernels in the metadata"
    return ks


def test_every_kernel_present(kernels):
    names = " ".join(k[".name"] for k in kernels)
    for fam in ("append_kernel", "append_fp8_kernel", "decode_kernel", "decode_balanced_kernel",
                "decode_multi_kernel", "merge_kernel", "merge_parts_kernel",
                "merge_pieces_kernel", "schedule_kernel", "copy_blocks_kernel"):
        assert fam in names, fam


def test_no_vector_spills_no_scratch(kernels):
    bad = [(k[".name"], k[".vgpr_spill_count"], k[".private_segment_fixed_size"])
           for k in kernels
           if k[".vgpr_spill_count"] != 0 or k[".private_segment_fixed_size"] != 0]
    assert not bad, f"kernels that spill vector registers or use scratch: {bad}"


def test_decode_kernels_fit_one_wave_per_simd(kernels):
    """The decode kernels are built for one wave per SIMD (512 registers:
    256 vector + 256 accumulation): a CU holds four waves, i.e. 4 / (waves
    per workgroup) workgroups, whose LDS must fit its 160 KiB."""
    for k in kernels:
        if "decode" not in k[".name"]:
            continue
        assert k[".vgpr_count"] <= 512, (k[".name"], k[".vgpr_count"])
        waves = max(1, k[".max_flat_workgroup_size"] // 64)
        groups = max(1, 4 // waves)
        assert groups * k[".group_segment_fixed_size"] <= 160 * 1024, k[".name"]
