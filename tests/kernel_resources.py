"""Per-kernel resources of the built library, read from its own gfx950 code
objects: the host library carries one clang offload bundle per translation
unit, the gfx950 entry of each is an ELF whose NT_AMDGPU_METADATA note
(msgpack) lists every kernel with its VGPR count and private (scratch) segment
size.  Used by the CPU tests to check properties the kernels' speed depends
on, without a GPU."""
import struct

import msgpack

_BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
_SHT_NOTE = 7
_NT_AMDGPU_METADATA = 32


def _bundle_entries(data: bytes):
    pos = data.find(_BUNDLE_MAGIC)
    while pos >= 0:
        count, = struct.unpack_from("<Q", data, pos + len(_BUNDLE_MAGIC))
        off = pos + len(_BUNDLE_MAGIC) + 8
        for _ in range(count):
            e_off, e_size, t_len = struct.unpack_from("<QQQ", data, off)
            triple = data[off + 24: off + 24 + t_len].decode()
            off += 24 + t_len
            yield triple, data[pos + e_off: pos + e_off + e_size]
        pos = data.find(_BUNDLE_MAGIC, pos + len(_BUNDLE_MAGIC))


def _elf_notes(elf: bytes):
    if elf[:4] != b"\x7fELF" or elf[4] != 2:   # 64-bit ELF only
        return
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum = struct.unpack_from("<HH", elf, 0x3A)
    for i in range(shnum):
        sh = shoff + i * shentsize
        sh_type, = struct.unpack_from("<I", elf, sh + 4)
        if sh_type != _SHT_NOTE:
            continue
        off, size = struct.unpack_from("<QQ", elf, sh + 0x18)
        p = off
        while p + 12 <= off + size:
            namesz, descsz, ntype = struct.unpack_from("<III", elf, p)
            name = elf[p + 12: p + 12 + namesz].rstrip(b"\0")
            desc = p + 12 + ((namesz + 3) & ~3)
            yield name, ntype, elf[desc: desc + descsz]
            p = desc + ((descsz + 3) & ~3)


def kernel_resources(lib_path: str, arch: str = "gfx950") -> dict:
    """{mangled kernel name: {"vgpr": n, "scratch": bytes per lane}}."""
    with open(lib_path, "rb") as f:
        data = f.read()
    out = {}
    for triple, blob in _bundle_entries(data):
        if not triple.endswith(arch):
            continue
        for name, ntype, desc in _elf_notes(blob):
            if name != b"AMDGPU" or ntype != _NT_AMDGPU_METADATA:
                continue
            for k in msgpack.unpackb(desc, raw=False).get("amdhsa.kernels", []):
                out[k[".name"]] = {"vgpr": k[".vgpr_count"],
                                   "scratch": k[".private_segment_fixed_size"]}
    return out
