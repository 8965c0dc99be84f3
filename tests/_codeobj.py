"""Kernel resource records of the gfx950 code objects inside a HIP shared
library built here (test infrastructure).

A HIP library carries its device code in the .hip_fatbin section as clang
offload bundles: the magic "__CLANG_OFFLOAD_BUNDLE__", an entry count, then
per entry (offset, size, target-triple length, triple), offsets relative to
the bundle start.  Each amdgcn entry is an ELF code object whose note of type
NT_AMDGPU_METADATA (32, owner "AMDGPU") holds msgpack metadata with one
record per kernel: name, VGPR/AGPR counts, spill counts and the per-lane
private (scratch) segment size.
"""
from __future__ import annotations

import struct

import msgpack

MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NT_AMDGPU_METADATA = 32


def _bundles(blob: bytes):
    pos = blob.find(MAGIC)
    while pos >= 0:
        (count,) = struct.unpack_from("<Q", blob, pos + len(MAGIC))
        q = pos + len(MAGIC) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", blob, q)
            q += 24
            triple = blob[q:q + tlen].decode()
            q += tlen
            yield triple, blob[pos + off:pos + off + size]
        pos = blob.find(MAGIC, q)


def _notes(elf: bytes):
    assert elf[:4] == b"\x7fELF" and elf[4] == 2, "64-bit ELF expected"
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum = struct.unpack_from("<HH", elf, 0x3A)
    for i in range(shnum):
        sh = shoff + i * shentsize
        sh_type, = struct.unpack_from("<I", elf, sh + 4)
        if sh_type != 7:  # SHT_NOTE
            continue
        off, size = struct.unpack_from("<QQ", elf, sh + 0x18)
        p, end = off, off + size
        while p + 12 <= end:
            namesz, descsz, ntype = struct.unpack_from("<III", elf, p)
            p += 12
            name = elf[p:p + namesz].rstrip(b"\0")
            p += (namesz + 3) & ~3
            desc = elf[p:p + descsz]
            p += (descsz + 3) & ~3
            yield name, ntype, desc


def kernel_records(lib_path: str, arch: str = "gfx950") -> list[dict]:
    """One metadata record per kernel of every `arch` code object in the library."""
    with open(lib_path, "rb") as f:
        blob = f.read()
    out = []
    for triple, obj in _bundles(blob):
        if not triple.startswith("hip") or arch not in triple:
            continue
        for name, ntype, desc in _notes(obj):
            if name == b"AMDGPU" and ntype == NT_AMDGPU_METADATA:
                meta = msgpack.unpackb(desc, raw=False)
                out.extend(meta.get("amdhsa.kernels", []))
    return out
