"""The build step that puts wait states after wide vector-memory stores (CPU).

A store of more than 8 bytes reads its data VGPRs after it issues; the pass must separate it from any
later write of those VGPRs by STORE_DATA_WAIT wait states, count s_nop n as n + 1, drain before labels and
branches, and change nothing but the added s_nop lines. The last test runs the checker over the code object
inside the built library.
"""
import os
import shutil
import subprocess

import pytest

from taylor_feature_map_amd import hazard_pad as hp

W = hp.STORE_DATA_WAIT
STORE = "\tbuffer_store_dwordx4 v[58:61], v82, s[36:39], s43 offen"


def _asm(*body):
    return "\n".join(["kern:", *body, "\ts_endpgm"])


def _nop_waits(text):
    return sum(i.waits for i in map(hp.parse_instruction, text.split("\n")) if i is not None and i.opcode == "s_nop")


def test_write_of_store_data_right_after_is_padded():
    src = _asm(STORE, "\tv_mul_f32_e32 v61, v65, v74")
    assert len(hp.check(src)) == 1
    rep = hp.pad(src)
    out = "\n".join(rep.lines)
    assert hp.check(out) == [] and hp.same_program(src, out)
    assert rep.sites == 1 and _nop_waits(out) == W


def test_address_register_is_protected_too():
    src = _asm(STORE, "\tv_add_u32_e32 v82, 64, v82")
    assert _nop_waits("\n".join(hp.pad(src).lines)) == W


def test_unrelated_write_narrow_store_and_reads_need_nothing():
    for body in ([STORE, "\tv_mul_f32_e32 v62, v65, v74"],                     # other register
                 ["\tbuffer_store_dwordx2 v[58:59], v82, s[36:39], s43 offen",  # 8 bytes
                  "\tv_mul_f32_e32 v59, v65, v74"],
                 [STORE, "\tv_mul_f32_e32 v70, v61, v74"],                      # reads v61 only
                 ["\tds_write_b128 v10, v[58:61]", "\tv_mov_b32_e32 v61, 0"]):   # LDS store
        src = _asm(*body)
        assert hp.check(src) == [] and hp.pad(src).lines == src.split("\n"), body


def test_distance_already_present_is_counted():
    # one instruction and s_nop 1 (two wait states) already separate them: one more is enough when W = 4
    src = _asm(STORE, "\tv_mov_b32_e32 v1, 0", "\ts_nop 1", "\tv_mov_b32_e32 v60, 0")
    out = "\n".join(hp.pad(src).lines)
    assert hp.check(out) == [] and _nop_waits(out) == 2 + max(W - 3, 0)
    far = _asm(STORE, *["\tv_mov_b32_e32 v1, 0"] * W, "\tv_mov_b32_e32 v60, 0")
    assert hp.check(far) == []


def test_global_store_and_dwordx3_are_wide():
    for st in ("\tglobal_store_dwordx4 v[2:3], v[58:61], off", "\tbuffer_store_dwordx3 v[58:60], v82, s[36:39], 0 offen"):
        src = _asm(st, "\tv_mov_b32_e32 v58, 0")
        assert len(hp.check(src)) == 1, st


def test_labels_and_branches_drain():
    src = "\n".join(["kern:", STORE, ".LBB0_1:", "\tv_mov_b32_e32 v1, 0", STORE, "\ts_cbranch_scc1 .LBB0_1",
                     "\ts_endpgm"])
    bad = hp.check(src)
    assert len(bad) == 2 and "label" in bad[0]
    rep = hp.pad(src)
    out = "\n".join(rep.lines)
    assert rep.drains == 2 and hp.check(out) == [] and hp.same_program(src, out)


def test_labels_are_only_symbols_at_line_start():
    assert hp.is_label(".LBB0_12:") and hp.is_label("_ZN5based3fooEv:   ; @_ZN5based3fooEv")
    assert hp.is_label("0000000000001900 <_ZN5based3fooEv>:")
    assert not hp.is_label("  - .args:") and not hp.is_label("      .name:           foo") and not hp.is_label("\ts_nop 0")


def test_same_program_rejects_any_other_change():
    src = _asm(STORE, "\tv_mul_f32_e32 v61, v65, v74")
    out = hp.pad(src).lines
    assert not hp.same_program(src, "\n".join(out[:-1]))
    changed = ["\tv_mul_f32_e32 v61, v66, v74" if "v_mul" in x else x for x in out]
    assert not hp.same_program(src, "\n".join(changed))
    assert not hp.same_program(src, "\n".join(["\tv_nop"] + out))


def test_bundle_reader():
    import struct
    payload = b"\x7fELF" + b"x" * 60
    triple = b"hipv4-amdgcn-amd-amdhsa--gfx950"
    host = b"host-x86_64-unknown-linux-gnu"
    header = b"__CLANG_OFFLOAD_BUNDLE__" + struct.pack("<Q", 2)
    entries_len = 2 * 24 + len(host) + len(triple)
    off = len(header) + entries_len
    blob = header + struct.pack("<QQQ", off, 0, len(host)) + host + struct.pack("<QQQ", off, len(payload), len(triple)) \
        + triple + payload
    got = hp.code_objects(b"junk" + blob + b"tail")
    assert got == {triple.decode(): payload}


LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "taylor_feature_map_amd", "libbased.so")
OBJDUMP = "/opt/rocm/lib/llvm/bin/llvm-objdump"


@pytest.mark.skipif(not (os.path.exists(LIB) and shutil.which(OBJDUMP)), reason="library or llvm-objdump missing")
def test_built_library_obeys_the_rule(tmp_path):
    with open(LIB, "rb") as f:
        objs = hp.code_objects(f.read())
    co = objs["hipv4-amdgcn-amd-amdhsa--gfx950"]
    path = tmp_path / "kernels.hsaco"
    path.write_bytes(co)
    dis = subprocess.run([OBJDUMP, "-d", str(path)], capture_output=True, text=True, check=True).stdout
    stores = [i for i in map(hp.parse_instruction, dis.split("\n")) if i is not None and i.is_wide_vmem_store]
    assert len(stores) > 50  # the fp32 output tiles, the state slots and the decode step
    assert hp.check(dis) == []
    # the same listing without its s_nop lines breaks the rule: the checker reads this disassembly
    stripped = "\n".join(x for x in dis.split("\n") if not ((i := hp.parse_instruction(x)) and i.opcode == "s_nop"))
    assert len(hp.check(stripped)) > 10


READELF = "/opt/rocm/lib/llvm/bin/llvm-readelf"


@pytest.mark.skipif(not (os.path.exists(LIB) and shutil.which(READELF)), reason="library or llvm-readelf missing")
def test_no_kernel_uses_scratch(tmp_path):
    """Every kernel keeps its values in registers and LDS: no private segment and no spills. (A query-side
    choice between two array elements once put the K = 8 read-out's arrays in scratch memory, stored and
    reloaded every chunk.)"""
    with open(LIB, "rb") as f:
        co = hp.code_objects(f.read())["hipv4-amdgcn-amd-amdhsa--gfx950"]
    path = tmp_path / "kernels.hsaco"
    path.write_bytes(co)
    notes = subprocess.run([READELF, "--notes", str(path)], capture_output=True, text=True, check=True).stdout
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
