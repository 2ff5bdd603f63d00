"""Fingerprints of the gfx950 kernels inside the built libmfl.so.

A measurement taken with hardware counters belongs to one build of one kernel.
This module finds that kernel's machine code in the library this repository
builds and hashes it, so that a stored counter record can be matched against
the library that is loaded now: an edit of comments or of host code leaves the
fingerprint unchanged, any change of the kernel's instructions or of its
resource descriptor changes it.

Layout walked (plain ELF64 parsing, no external tools): the host shared object
holds a ``.hip_fatbin`` section made of clang offload bundles; each bundle lists
(offset, size, target triple) entries, and the ``amdgcn-amd-amdhsa--gfx950``
entry is an AMDGPU code object (itself ELF64) whose symbol table names every
kernel (a function symbol: its instructions) and its kernel descriptor
(``<name>.kd``, 64 bytes: register counts, LDS size, launch settings).
"""
from __future__ import annotations

import hashlib
import struct

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
ARCH = "gfx950"
STT_FUNC, STT_OBJECT = 2, 1


def _sections(elf: bytes):
    """(name, offset, size, addr, link) of every section of an ELF64 image."""
    if elf[:4] != b"\x7fELF" or elf[4] != 2:
        raise ValueError("not an ELF64 image")
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    raw = []
    for i in range(shnum):
        base = shoff + i * shentsize
        name, typ, flags, addr, off, size, link = struct.unpack_from("<IIQQQQI", elf, base)
        raw.append((name, typ, addr, off, size, link))
    stroff = raw[shstrndx][3]

    def cstr(off):
        return elf[off:elf.index(b"\0", off)].decode()

    return [(cstr(stroff + n), off, size, addr, link, typ) for n, typ, addr, off, size, link in raw]


def _symbols(elf: bytes):
    """name -> (type, value, size) from the .symtab (or .dynsym) of an ELF64 image."""
    secs = _sections(elf)
    out = {}
    for name, off, size, _, link, typ in secs:
        if name not in (".symtab", ".dynsym"):
            continue
        stroff = secs[link][1]
        for i in range(size // 24):
            st_name, info, _, _, value, sz = struct.unpack_from("<IBBHQQ", elf, off + 24 * i)
            if st_name == 0:
                continue
            nm = elf[stroff + st_name:elf.index(b"\0", stroff + st_name)].decode()
            out.setdefault(nm, (info & 15, value, sz))
    return out


def _bytes_at(elf: bytes, secs, vaddr: int, size: int) -> bytes:
    for _, off, ssize, addr, _, typ in secs:
        if typ != 8 and addr <= vaddr < addr + ssize and addr != 0:   # 8: SHT_NOBITS
            start = off + vaddr - addr
            return elf[start:start + size]
    raise ValueError(f"address {vaddr:#x} not in any section")


def code_objects(lib_path: str):
    """The gfx950 code objects embedded in a host shared object."""
    data = open(lib_path, "rb").read()
    fat = [s for s in _sections(data) if s[0] == ".hip_fatbin"]
    if not fat:
        raise ValueError(f"{lib_path}: no .hip_fatbin section")
    _, off, size, _, _, _ = fat[0]
    blob = data[off:off + size]
    objs = []
    pos = blob.find(BUNDLE_MAGIC)
    while pos >= 0:
        n = struct.unpack_from("<Q", blob, pos + 24)[0]
        p = pos + 32
        for _ in range(n):
            eoff, esize, tlen = struct.unpack_from("<QQQ", blob, p)
            triple = blob[p + 24:p + 24 + tlen].decode()
            p += 24 + tlen
            if triple.endswith("--" + ARCH):
                objs.append(blob[pos + eoff:pos + eoff + esize])
        pos = blob.find(BUNDLE_MAGIC, pos + 32)
    return objs


def kernels(lib_path: str):
    """mangled kernel name -> sha256 of its instructions and its kernel
    descriptor (without the descriptor's entry-offset field, which only says
    where the code was placed)."""
    out = {}
    for obj in code_objects(lib_path):
        secs = _sections(obj)
        syms = _symbols(obj)
        for name, (typ, value, size) in syms.items():
            kd = syms.get(name + ".kd")
            if typ != STT_FUNC or kd is None or size == 0:
                continue
            code = _bytes_at(obj, secs, value, size)
            desc = _bytes_at(obj, secs, kd[1], 64)
            h = hashlib.sha256()
            h.update(code)
            h.update(desc[:16] + desc[24:])
            out[name] = h.hexdigest()
    return out


def kernel_digest(lib_path: str, pattern: str):
    """(mangled name, digest) of the one kernel whose mangled name contains
    ``pattern``; ValueError if none or several match."""
    found = [(n, d) for n, d in kernels(lib_path).items() if pattern in n]
    if len(found) != 1:
        raise ValueError(f"{len(found)} kernels match {pattern!r}")
    return found[0]
