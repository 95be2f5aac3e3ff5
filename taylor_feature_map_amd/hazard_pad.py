"""Build step: pads the gfx950 device assembly after wide vector-memory stores.

A vector-memory store of more than 8 bytes (buffer/global/flat/scratch `_dwordx3`, `_dwordx4`) reads its
data VGPRs after it issues, so an instruction that overwrites one of them right behind it can change
what is stored. The compiler pads this case only for stores whose offset is not an SGPR. The read-out
kernels store fp32 output tiles with buffer_store_dwordx4 and the row offset in an SGPR, and the compiler
let the next tile's scaling overwrite the data registers in the very next instruction. On MI355X the last
dword (value column 4g + 3) of lanes 12-15 was then now and then stored with the next tile's value:
wrong fp32 outputs that changed from run to run. bf16 tiles are 8-byte stores and were never affected.

`pad()` walks every function in program order and inserts `s_nop` so that at least `STORE_DATA_WAIT`
wait states separate such a store from any later instruction that writes one of the store's VGPR
operands (data or address). One instruction counts one wait state and `s_nop n` counts n + 1. Control
flow is handled by draining: before every branch and every label, nops are added until no wide store
is still inside its window, so a block starts clean however it is entered.

`check()` applies the same rule to a listing (the assembly, or `llvm-objdump -d` of a code object) and
returns the violations; the build runs it on its own output and a test runs it on the code object
inside the built library. `code_objects()` pulls that code object out of the library.
"""
from __future__ import annotations

import re
import struct
from dataclasses import dataclass, field
from typing import List, Optional, Set

# The hazard needs one wait state; three more are a margin (the cost is a few nops per output tile).
STORE_DATA_WAIT = 4

_REG = re.compile(r"(?<![\w.])v(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
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

    def vgprs(self) -> Set[int]:
        out: Set[int] = set()
        for o in self.operands:
            out |= _vgprs(o)
        return out

    def written(self) -> Set[int]:
        """VGPRs the instruction may write: its first operand, unless it is a store."""
        if _STORE.match(self.opcode) or not self.operands:
            return set()
        return _vgprs(self.operands[0])


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
    """Wide stores issued less than STORE_DATA_WAIT wait states ago, with the VGPRs they read."""

    def __init__(self) -> None:
        self.pending: List[List] = []  # [vgprs, age]

    def need(self, ins: Instr) -> int:
        written = ins.written()
        if not written:
            return 0
        return max([STORE_DATA_WAIT - age for regs, age in self.pending if regs & written] + [0])

    def drain_need(self) -> int:
        return max([STORE_DATA_WAIT - age for _, age in self.pending] + [0])

    def advance(self, waits: int) -> None:
        for p in self.pending:
            p[1] += waits
        self.pending = [p for p in self.pending if p[1] < STORE_DATA_WAIT]

    def issue(self, ins: Instr) -> None:
        self.advance(ins.waits)
        if ins.is_wide_vmem_store:
            self.pending.append([ins.vgprs(), 0])
        if ins.is_end or ins.is_branch:
            self.pending = []


def _nops(n: int) -> List[str]:
    out = []
    while n > 0:
        k = min(n, 8)
        out.append(f"\ts_nop {k - 1}")
        n -= k
    return out


@dataclass
class PadReport:
    sites: int = 0
    drains: int = 0
    waits_added: int = 0
    lines: List[str] = field(default_factory=list)


def pad(asm: str) -> PadReport:
    """The padded assembly (in `.lines`) and how much was added."""
    rep = PadReport()
    tr = _Tracker()
    for line in asm.split("\n"):
        if is_label(line):
            n = tr.drain_need()
            if n:
                rep.lines += _nops(n)
                rep.drains += 1
                rep.waits_added += n
            tr.pending = []
            rep.lines.append(line)
            continue
        ins = parse_instruction(line)
        if ins is not None:
            n = tr.drain_need() if ins.is_branch else tr.need(ins)
            if n:
                rep.lines += _nops(n)
                tr.advance(n)
                rep.waits_added += n
                if ins.is_branch:
                    rep.drains += 1
                else:
                    rep.sites += 1
            tr.issue(ins)
        rep.lines.append(line)
    return rep


def check(listing: str) -> List[str]:
    """Every place in a listing where the rule is broken. Disassembly has no labels: it is then checked
    as one straight line, and every branch must find no wide store inside its window."""
    bad: List[str] = []
    tr = _Tracker()
    for no, line in enumerate(listing.split("\n"), 1):
        if is_label(line):
            if tr.drain_need():
                bad.append(f"line {no}: label reached inside a wide store's window: {line.strip()}")
            tr.pending = []
            continue
        ins = parse_instruction(line)
        if ins is None:
            continue
        n = tr.drain_need() if ins.is_branch else tr.need(ins)
        if n:
            bad.append(f"line {no}: {n} wait states short before: {line.strip()}")
        tr.issue(ins)
    return bad


def same_program(original: str, padded: str) -> bool:
    """True when `padded` is `original` with only s_nop lines added: every original line is there,
    unchanged and in order, and every extra line is an s_nop."""
    orig = original.split("\n")
    i = 0
    for line in padded.split("\n"):
        if i < len(orig) and line == orig[i]:
            i += 1
            continue
        ins = parse_instruction(line)
        if ins is None or ins.opcode != "s_nop":
            return False
    return i == len(orig)


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
