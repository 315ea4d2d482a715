"""Register and scratch use of every kernel in the built library, read from the gfx950 code
objects that hipcc embedded in libpa.so (no GPU needed).

Each compiled source leaves one offload bundle in the library; its gfx950 entry is an AMDGPU ELF
whose metadata note (msgpack) lists every kernel with its private-segment (scratch) size, spill
counts and register counts."""
import struct

import msgpack
import pytest

from paged_kv_cache_177_amd.build import LIB

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NT_AMDGPU_METADATA = 32
SHT_NOTE = 7


def _code_objects(data: bytes):
    """The gfx950 code objects of every offload bundle in `data`."""
    at = data.find(BUNDLE_MAGIC)
    while at >= 0:
        (n,) = struct.unpack_from("<Q", data, at + len(BUNDLE_MAGIC))
        off = at + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            e_off, e_size, t_len = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + t_len].decode()
            off += t_len
            if triple.endswith("gfx950") and e_size > 0:
                yield data[at + e_off:at + e_off + e_size]
        at = data.find(BUNDLE_MAGIC, at + 1)


def _kernels(elf: bytes):
    """The `amdhsa.kernels` metadata entries of one code object."""
    assert elf[:4] == b"\x7fELF" and elf[4] == 2  # ELF64
    e_shoff, = struct.unpack_from("<Q", elf, 0x28)
    e_shentsize, e_shnum = struct.unpack_from("<HH", elf, 0x3A)
    out = []
    for i in range(e_shnum):
        sh = e_shoff + i * e_shentsize
        sh_type, = struct.unpack_from("<I", elf, sh + 4)
        if sh_type != SHT_NOTE:
            continue
        s_off, s_size = struct.unpack_from("<QQ", elf, sh + 0x18)
        p, end = s_off, s_off + s_size
        while p + 12 <= end:
            namesz, descsz, ntype = struct.unpack_from("<III", elf, p)
            name = elf[p + 12:p + 12 + namesz]
            desc_at = p + 12 + ((namesz + 3) & ~3)
            if ntype == NT_AMDGPU_METADATA and name.rstrip(b"\0") == b"AMDGPU":
                meta = msgpack.unpackb(elf[desc_at:desc_at + descsz], raw=False)
                out.extend(meta["amdhsa.kernels"])
            p = desc_at + ((descsz + 3) & ~3)
    return out


@pytest.fixture(scope="module")
def kernels():
    with open(LIB, "rb") as f:
        data = f.read()
    ks = [k for co in _code_objects(data) for k in _kernels(co)]
    assert ks, "no gfx950 kernels found in the library"
    return ks


def test_no_kernel_uses_scratch_memory(kernels):
    """No kernel instance keeps anything in scratch memory: no private segment and no dynamic
    stack. Register-to-register spills are allowed (scalar registers parked in vector-register
    lanes, and the fp32 instances for groups of 8 heads parking vector registers in accumulation
    registers): they cost no memory traffic."""
    bad = [(k[".name"], k.get(".private_segment_fixed_size")) for k in kernels
           if k.get(".private_segment_fixed_size", 0) or k.get(".uses_dynamic_stack", False)]
    assert not bad, bad


def test_bf16_split_grid_keeps_three_workgroups_per_cu(kernels):
    """The bf16 split-grid decode instances for groups of up to 4 query heads fit in 168
    registers (the metadata's count covers the accumulation registers too), so 3 workgroups of 4
    waves fit on a CU: the occupancy their launches are held to."""
    grid = [k for k in kernels if "decode_vector_kernelIDF16b" in k[".name"]
            and any(f"ELi{g}ELb" in k[".name"] for g in (1, 2, 4))]
    assert grid
    for k in grid:
        assert k[".vgpr_count"] <= 168, (k[".name"], k[".vgpr_count"], k.get(".agpr_count"))
