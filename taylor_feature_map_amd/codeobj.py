"""Checks on the gfx950 code object inside the built library (used by tests and the measurement).

A vector-memory store of more than 8 bytes (buffer/global/flat/scratch `_dwordx3`, `_dwordx4`) reads its
data VGPRs after it issues, so an instruction that overwrites one of them right behind it can change what
is stored; the hardware needs one wait state between them. The compiler inserts it, except for buffer
stores whose scalar offset is an SGPR: such a store once let the next output tile's products overwrite
the data of fp32 output tiles, which then changed from run to run. The kernels therefore pass a constant
scalar offset to every wide buffer store, and these checks hold the built code to that:
- `wide_stores_with_sgpr_offset()` lists the wide buffer stores whose scalar offset is an SGPR;
- `check()` lists every place where fewer than `wait` wait states separate a wide store from a later
  VALU write of one of its data VGPRs (one instruction counts one wait state, `s_nop n` counts n + 1;
  labels and branches must be reached with no wide store inside its window). Loads that write those
  VGPRs do so only when their data returns, long after the store has read them.
`code_objects()` pulls the device code objects out of the library and `text_digest()` hashes the
instruction bytes of the gfx950 one (independent of the build directory, which other sections record).
"""
from __future__ import annotations

import hashlib
import re
import struct
from dataclasses import dataclass
from typing import List, Optional, Set

# Wait states the hardware needs between a wide store and a write of its data VGPRs.
STORE_DATA_WAIT = 1
GFX950 = "hipv4-amdgcn-amd-amdhsa--gfx950"

_REG = re.compile(r"(?<![\w.])v(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_SREG = re.compile(r"^(s\d+|s\[\d+:\d+\]|m0|vcc_lo|vcc_hi|ttmp\d+)$")
_STORE = re.compile(r"^(ds_write|ds_store|buffer_store|global_store|flat_store|scratch_store)")
_WIDE_VMEM_STORE = re.compile(r"^(buffer|global|flat|scratch)_store_(dwordx3|dwordx4|b96|b128)\b")
_BRANCH = re.compile(r"^(s_branch|s_cbranch|s_setpc|s_swappc|s_call)")
_END = re.compile(r"^(s_endpgm|s_code_end)")
_OPCODE = re.compile(r"^[sv]_|^(ds|buffer|global|flat|scratch|exp|image)_")


def _vgprs(text: str) -> Set[int]:
    """VGPR numbers named in an operand string."""
    out: Set[int] = set()
    for m in _REG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _split_operands(rest: str) -> List[str]:
    ops, depth, cur = [], 0, []
    for ch in rest:
        depth += (ch == "[") - (ch == "]")
        if ch == "," and depth == 0:
            ops.append("".join(cur).strip())
            cur = []
        else:
            cur.append(ch)
    if "".join(cur).strip():
        ops.append("".join(cur).strip())
    return ops


@dataclass
class Instr:
    opcode: str
    operands: List[str]
    waits: int

    @property
    def is_branch(self) -> bool:
        return bool(_BRANCH.match(self.opcode))

    @property
    def is_end(self) -> bool:
        return bool(_END.match(self.opcode))

    @property
    def is_wide_vmem_store(self) -> bool:
        return bool(_WIDE_VMEM_STORE.match(self.opcode))

    def data_vgprs(self) -> Set[int]:
        """The VGPRs holding a store's data: the first operand of a buffer or scratch store, the second
        of a global or flat store (which lead with the address)."""
        if not _STORE.match(self.opcode) or not self.operands:
            return set()
        idx = 1 if self.opcode.startswith(("global_", "flat_")) else 0
        return _vgprs(self.operands[idx]) if len(self.operands) > idx else set()

    def valu_written(self) -> Set[int]:
        """VGPRs a VALU instruction writes (its first operand)."""
        if not self.opcode.startswith("v_") or not self.operands:
            return set()
        return _vgprs(self.operands[0])

    def scalar_offset(self) -> Optional[str]:
        """The scalar offset operand of a buffer store (data, vaddr, rsrc, soffset, modifiers...)."""
        if not self.opcode.startswith("buffer_store") or len(self.operands) < 4:
            return None
        return self.operands[3].split()[0]


def parse_instruction(text: str) -> Optional[Instr]:
    """The instruction on one line of assembly or disassembly; None for labels, directives, comments."""
    s = text.split(";")[0].split("//")[0].strip()
    if not s or s.startswith(".") or s.endswith(":"):
        return None
    opcode = s.split()[0]
    if not _OPCODE.match(opcode):
        return None
    rest = s[len(opcode):]
    waits = 1
    if opcode == "s_nop":
        arg = rest.strip()
        waits = (int(arg, 0) if arg else 0) + 1
    return Instr(opcode, _split_operands(rest), waits)


_LABEL = re.compile(r"^[A-Za-z_.$][\w.$]*:\s*$")          # assembly: a symbol at the start of the line
_DIS_LABEL = re.compile(r"^[0-9a-fA-F]+ <[^>]+>:\s*$")     # llvm-objdump: address <symbol>:


def is_label(text: str) -> bool:
    """A label line of assembly or disassembly (never an indented line, such as a YAML key in the
    metadata block)."""
    s = text.split(";")[0].rstrip()
    return bool(_LABEL.match(s) or _DIS_LABEL.match(s))


class _Tracker:
    """Wide stores issued less than `wait` wait states ago, with the VGPRs they read."""

    def __init__(self, wait: int) -> None:
        self.wait = wait
        self.pending: List[List] = []  # [vgprs, age]

    def need(self, ins: Instr) -> int:
        written = ins.valu_written()
        if not written:
            return 0
        return max([self.wait - age for regs, age in self.pending if regs & written] + [0])

    def drain_need(self, own: int = 0) -> int:
        """Wait states still needed when control leaves here; `own` counts those of the branch itself."""
        return max([self.wait - age - own for _, age in self.pending] + [0])

    def issue(self, ins: Instr) -> None:
        for p in self.pending:
            p[1] += ins.waits
        self.pending = [p for p in self.pending if p[1] < self.wait]
        if ins.is_wide_vmem_store:
            self.pending.append([ins.data_vgprs(), 0])
        if ins.is_end or ins.is_branch:
            self.pending = []


def check(listing: str, wait: int = STORE_DATA_WAIT) -> List[str]:
    """Every place in a listing where fewer than `wait` wait states separate a wide store from a VALU
    write of its data VGPRs. Disassembly has no labels: it is then checked as one straight line, and every branch must
    find no wide store inside its window."""
    bad: List[str] = []
    tr = _Tracker(wait)
    for no, line in enumerate(listing.split("\n"), 1):
        if is_label(line):
            if tr.drain_need():
                bad.append(f"line {no}: label reached inside a wide store's window: {line.strip()}")
            tr.pending = []
            continue
        ins = parse_instruction(line)
        if ins is None:
            continue
        n = tr.drain_need(ins.waits) if ins.is_branch else tr.need(ins)
        if n:
            bad.append(f"line {no}: {n} wait states short before: {line.strip()}")
        tr.issue(ins)
    return bad


def wide_stores_with_sgpr_offset(listing: str) -> List[str]:
    """The wide buffer stores of a listing whose scalar offset is an SGPR."""
    out = []
    for line in listing.split("\n"):
        ins = parse_instruction(line)
        if ins is not None and ins.is_wide_vmem_store:
            so = ins.scalar_offset()
            if so is not None and _SREG.match(so):
                out.append(line.strip())
    return out


_BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def code_objects(lib_bytes: bytes) -> dict:
    """The device code objects embedded in a built shared library, keyed by bundle target.

    A HIP fat binary is an uncompressed clang offload bundle: the magic string, the entry count, then per
    entry its offset and size (from the bundle's start) and its target triple, all little-endian 64-bit
    fields apart from the triple's bytes.
    """
    out = {}
    pos = lib_bytes.find(_BUNDLE_MAGIC)
    while pos >= 0:
        cur = pos + len(_BUNDLE_MAGIC)
        (count,) = struct.unpack_from("<Q", lib_bytes, cur)
        cur += 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", lib_bytes, cur)
            cur += 24
            triple = lib_bytes[cur:cur + tlen].decode()
            cur += tlen
            if size:
                out[triple] = lib_bytes[pos + off:pos + off + size]
        pos = lib_bytes.find(_BUNDLE_MAGIC, cur)
    return out


def elf_section(elf: bytes, name: str) -> bytes:
    """The bytes of section `name` of a 64-bit little-endian ELF file (a code object)."""
    if elf[:4] != b"\x7fELF" or elf[4] != 2 or elf[5] != 1:
        raise ValueError("not a 64-bit little-endian ELF file")
    e_shoff, = struct.unpack_from("<Q", elf, 0x28)
    e_shentsize, e_shnum, e_shstrndx = struct.unpack_from("<HHH", elf, 0x3A)

    def header(i):
        # sh_name, sh_type, sh_flags, sh_addr, sh_offset, sh_size
        return struct.unpack_from("<IIQQQQ", elf, e_shoff + i * e_shentsize)

    str_off, str_size = header(e_shstrndx)[4:6]
    strtab = elf[str_off:str_off + str_size]
    for i in range(e_shnum):
        sh_name, _, _, _, off, size = header(i)
        end = strtab.index(b"\0", sh_name)
        if strtab[sh_name:end].decode() == name:
            return elf[off:off + size]
    raise KeyError(name)


def text_digest(lib_path: str) -> Optional[str]:
    """SHA-256 of the instruction bytes (.text) of the gfx950 code object inside a built library, or None
    without one. It changes whenever the device code does (kernel source, compiler flags) and not for
    comments, host code or the directory the library was built in."""
    try:
        with open(lib_path, "rb") as f:
            co = code_objects(f.read()).get(GFX950)
    except OSError:
        return None
    if not co:
        return None
    return hashlib.sha256(elf_section(co, ".text")).hexdigest()
