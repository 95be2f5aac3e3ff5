"""The built gfx950 code object (CPU): wide-store rule, no scratch, a digest independent of the build
directory.

A store of more than 8 bytes reads its data VGPRs after it issues; a VALU write of them needs one wait
state behind it. The compiler pads this except for buffer stores whose scalar offset is an SGPR, so the
kernels keep that offset constant; these tests hold the built code to both.
"""
import os
import shutil
import struct
import subprocess

import pytest

from taylor_feature_map_amd import codeobj as co

STORE = "\tbuffer_store_dwordx4 v[58:61], v82, s[36:39], 0 offen"


def _asm(*body):
    return "\n".join(["kern:", *body, "\ts_endpgm"])


def test_valu_write_of_store_data_right_after_is_flagged():
    assert len(co.check(_asm(STORE, "\tv_mul_f32_e32 v61, v65, v74"))) == 1
    assert co.check(_asm(STORE, "\ts_nop 0", "\tv_mul_f32_e32 v61, v65, v74")) == []
    assert len(co.check(_asm(STORE, "\ts_nop 0", "\tv_mul_f32_e32 v61, v65, v74"), wait=3)) == 1


def test_address_registers_loads_narrow_stores_and_reads_are_not_flagged():
    for body in ([STORE, "\tv_add_u32_e32 v82, 64, v82"],                       # address register
                 [STORE, "\tds_read_b64_tr_b16 v[60:61], v99 offset:1536"],     # a load's data comes back later
                 ["\tbuffer_store_dwordx2 v[58:59], v82, s[36:39], 0 offen",   # 8 bytes
                  "\tv_mul_f32_e32 v59, v65, v74"],
                 [STORE, "\tv_mul_f32_e32 v70, v61, v74"],                      # reads v61 only
                 ["\tds_write_b128 v10, v[58:61]", "\tv_mov_b32_e32 v61, 0"]):   # LDS store
        assert co.check(_asm(*body)) == [], body


def test_global_store_data_is_its_second_operand():
    src = _asm("\tglobal_store_dwordx4 v[2:3], v[58:61], off", "\tv_mov_b32_e32 v58, 0")
    assert len(co.check(src)) == 1
    assert co.check(_asm("\tglobal_store_dwordx4 v[2:3], v[58:61], off", "\tv_mov_b32_e32 v2, 0")) == []


def test_labels_and_branches_drain():
    src = "\n".join(["kern:", STORE, ".LBB0_1:", "\tv_mov_b32_e32 v1, 0", STORE, "\ts_cbranch_scc1 .LBB0_1",
                     "\ts_endpgm"])
    bad = co.check(src)
    assert len(bad) == 1 and "label" in bad[0]  # the branch is itself the one wait state
    assert len(co.check(src, wait=2)) == 2


def test_labels_are_only_symbols_at_line_start():
    assert co.is_label(".LBB0_12:") and co.is_label("_ZN5based3fooEv:   ; @_ZN5based3fooEv")
    assert co.is_label("0000000000001900 <_ZN5based3fooEv>:")
    assert not co.is_label("  - .args:") and not co.is_label("      .name:           foo")
    assert not co.is_label("\ts_nop 0")


def test_scalar_offset_of_buffer_stores():
    sg = co.wide_stores_with_sgpr_offset(_asm("\tbuffer_store_dwordx4 v[94:97], v173, s[36:39], s43 offen",
                                              STORE, "\tbuffer_store_dwordx2 v[1:2], v3, s[36:39], s4 offen"))
    assert len(sg) == 1 and "s43" in sg[0]


def test_bundle_and_elf_readers():
    # a minimal ELF with a section header table: null, .text, .shstrtab
    shstr = b"\0.text\0.shstrtab\0"
    text = b"\x01\x02\x03\x04"
    hdr_size, sh_size = 64, 64
    text_off = hdr_size
    str_off = text_off + len(text)
    sh_off = str_off + len(shstr)
    ident = b"\x7fELF" + bytes([2, 1, 1]) + bytes(9)
    ehdr = ident + struct.pack("<HHIQQQIHHHHHH", 3, 224, 1, 0, 0, sh_off, 0, hdr_size, 0, 0, sh_size, 3, 2)
    sects = bytes(sh_size)
    sects += struct.pack("<IIQQQQIIQQ", 1, 1, 6, 0, text_off, len(text), 0, 0, 4, 0)
    sects += struct.pack("<IIQQQQIIQQ", 7, 3, 0, 0, str_off, len(shstr), 0, 0, 1, 0)
    elf = ehdr + text + shstr + sects
    assert co.elf_section(elf, ".text") == text
    triple = b"hipv4-amdgcn-amd-amdhsa--gfx950"
    host = b"host-x86_64-unknown-linux-gnu"
    header = b"__CLANG_OFFLOAD_BUNDLE__" + struct.pack("<Q", 2)
    off = len(header) + 2 * 24 + len(host) + len(triple)
    blob = header + struct.pack("<QQQ", off, 0, len(host)) + host + struct.pack("<QQQ", off, len(elf), len(triple)) \
        + triple + elf
    assert co.code_objects(b"junk" + blob + b"tail") == {triple.decode(): elf}


LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "taylor_feature_map_amd", "libbased.so")
OBJDUMP = "/opt/rocm/lib/llvm/bin/llvm-objdump"
READELF = "/opt/rocm/lib/llvm/bin/llvm-readelf"


def _code_object(tmp_path):
    with open(LIB, "rb") as f:
        data = co.code_objects(f.read())[co.GFX950]
    path = tmp_path / "kernels.hsaco"
    path.write_bytes(data)
    return path


@pytest.mark.skipif(not (os.path.exists(LIB) and shutil.which(OBJDUMP)), reason="library or llvm-objdump missing")
def test_built_library_obeys_the_store_rule(tmp_path):
    dis = subprocess.run([OBJDUMP, "-d", str(_code_object(tmp_path))], capture_output=True, text=True,
                         check=True).stdout
    stores = [i for i in map(co.parse_instruction, dis.split("\n")) if i is not None and i.is_wide_vmem_store]
    assert len(stores) > 50  # the fp32 output tiles, the state slots and the decode step
    assert co.wide_stores_with_sgpr_offset(dis) == []
    assert co.check(dis) == []
    # the same listing without its s_nop lines breaks the rule: the compiler's padding is what the
    # checker sees
    stripped = "\n".join(x for x in dis.split("\n") if not ((i := co.parse_instruction(x)) and i.opcode == "s_nop"))
    assert len(co.check(stripped)) > 10


@pytest.mark.skipif(not (os.path.exists(LIB) and shutil.which(READELF)), reason="library or llvm-readelf missing")
def test_no_kernel_uses_scratch(tmp_path):
    """Every kernel keeps its values in registers and LDS: no private segment and no spills. (A query-side
    choice between two array elements once put the K = 8 read-out's arrays in scratch memory, stored and
    reloaded every chunk.)"""
    notes = subprocess.run([READELF, "--notes", str(_code_object(tmp_path))], capture_output=True, text=True,
                           check=True).stdout
    kernels, fields = [], {}
    for line in notes.split("\n"):
        s = line.strip()
        if s.startswith(".name:"):
            kernels.append(s.split(":", 1)[1].strip())
        for key in ("private_segment_fixed_size", "sgpr_spill_count", "vgpr_spill_count"):
            if s.startswith(f".{key}:"):
                fields.setdefault(key, []).append(int(s.split(":", 1)[1]))
    assert len(kernels) >= 10
    for key, vals in fields.items():
        assert len(vals) == len(kernels) and all(v == 0 for v in vals), (key, list(zip(kernels, vals)))


@pytest.mark.skipif(not os.path.exists(LIB), reason="library missing")
def test_text_digest_is_the_instruction_bytes():
    d = co.text_digest(LIB)
    assert d is not None and len(d) == 64
    with open(LIB, "rb") as f:
        elf = co.code_objects(f.read())[co.GFX950]
    import hashlib
    assert d == hashlib.sha256(co.elf_section(elf, ".text")).hexdigest()
