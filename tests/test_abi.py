"""CPU checks of the C ABI: the library loads, exports every symbol include/based.h declares, and rejects
bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import math
import os
import re

import pytest

from taylor_feature_map_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "based.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(based_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    syms = header_symbols()
    assert syms, "no declarations found"
    assert sorted(_lib.SIGNATURES) == syms


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in header_symbols():
        assert hasattr(lib, name), name
    assert lib.based_abi_version() == 4
    for s in range(6):
        assert lib.based_status_string(s)
    assert lib.based_kernel_name(0) == b"based_segment_state_kernel"
    assert lib.based_kernel_name(1) == b"based_segment_scan_kernel"
    assert lib.based_kernel_name(2) == b"based_chunk_readout_kernel"
    assert lib.based_kernel_name(3) is None
    assert lib.based_kernel_name(7) is None


FAKE = 0x10000  # aligned non-null address; validation rejects the call before it is ever dereferenced


def call(q=FAKE, k=FAKE, v=FAKE, B=1, T=64, H=2, K=16, V=64, scale=math.nan, out=0x80000000, dt=0):
    lib = _lib.lib()
    return lib.based_forward(q, k, v, B, T, H, K, V, scale, out, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(out=0), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(B=0), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(T=0), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(H=-1), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(K=12), _lib.BASED_ERR_UNSUPPORTED),
    (dict(V=96), _lib.BASED_ERR_UNSUPPORTED),
    (dict(V=1024), _lib.BASED_ERR_UNSUPPORTED),
    (dict(T=1 << 20, H=16, V=128), _lib.BASED_ERR_UNSUPPORTED),  # rows exceed a 32-bit buffer range
    (dict(scale=math.inf), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(scale=-math.inf), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 2), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(dt=7), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(out=FAKE), _lib.BASED_ERR_INVALID_ARGUMENT),  # out overlaps the inputs
])
def test_invalid_arguments_rejected_on_host(kw, status):
    assert call(**kw) == status
    assert _lib.lib().based_last_error_detail()


def test_workspace_checks():
    lib = _lib.lib()
    need = lib.based_forward_workspace_bytes(4, 8192, 16, 16, 64)
    assert need > 0
    st = lib.based_forward_ws(FAKE, FAKE, FAKE, 4, 8192, 16, 16, 64, math.nan, 0x8000000000, 0, None, 0, None)
    assert st == _lib.BASED_ERR_WORKSPACE_TOO_SMALL
    st = lib.based_forward_ws(FAKE, FAKE, FAKE, 4, 8192, 16, 16, 64, math.nan, 0x8000000000, 0, 0x100000000,
                              need - 1, None)
    assert st == _lib.BASED_ERR_WORKSPACE_TOO_SMALL
    assert lib.based_forward_workspace_bytes(1, 64, 1, 12, 64) == 0


def test_plan():
    from taylor_feature_map_amd import plan
    g, L, ws = plan(4, 8192, 16, 16, 64)
    assert L % 32 == 0 and g == -(-8192 // L) and g * 64 >= 512
    assert g == 8  # 64 (b, h) items x 8 segments x 4 waves = 2048 waves: two per SIMD, no more
    g, L, ws = plan(1, 65000, 16, 16, 64)
    assert (g - 1) * L < 65000 <= g * L
    g, L, ws = plan(1, 1 << 20, 1, 16, 64)
    assert g > 16 and (g - 1) * L < (1 << 20) <= g * L
    g, L, ws = plan(1, 100, 1, 8, 64, segment_len=1000)
    assert g == 1 and ws == 0
    g, L, ws = plan(1, 100, 1, 8, 64, segment_len=33)
    assert L == 64 and g == 2


def test_feature_dim():
    lib = _lib.lib()
    assert lib.based_feature_dim(16) == 273 and lib.based_feature_dim(8) == 73


S_IN, Z_IN, S_OUT, Z_OUT = 0x2000000000, 0x3000000000, 0x4000000000, 0x5000000000


def call_state(s_in=None, z_in=None, s_out=None, z_out=None, K=16, V=64, T=64, out=0x80000000, ws=None, ws_bytes=0):
    lib = _lib.lib()
    return lib.based_forward_state(FAKE, FAKE, FAKE, 1, T, 2, K, V, math.nan, out, 0, s_in, z_in, s_out, z_out,
                                   ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(s_in=S_IN),                                    # state without its normaliser
    dict(z_out=Z_OUT),                                  # normaliser out without the state out
    dict(s_in=S_IN + 4, z_in=Z_IN),                     # misaligned
    dict(s_out=S_OUT, z_out=Z_OUT, out=S_OUT + 64),     # out overlaps state_out
    dict(s_in=S_IN, z_in=Z_IN, s_out=S_IN, z_out=Z_OUT),  # state_out aliases state_in
    dict(s_out=S_OUT, z_out=S_OUT + 256),               # state_out and norm_out overlap
])
def test_forward_state_rejects_bad_state_arguments(kw):
    assert call_state(**kw) == _lib.BASED_ERR_INVALID_ARGUMENT


def test_forward_state_rejects_unsupported_shape():
    assert call_state(s_out=S_OUT, z_out=Z_OUT, K=12) == _lib.BASED_ERR_UNSUPPORTED


def call_decode(q=FAKE, state=S_IN, norm=Z_IN, K=16, V=64, out=0x80000000, scale=math.nan):
    lib = _lib.lib()
    return lib.based_decode_step(q, FAKE, FAKE, 2, 4, K, V, scale, state, norm, out, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(state=0), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(norm=Z_IN + 8), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(K=4), _lib.BASED_ERR_UNSUPPORTED),
    (dict(V=100), _lib.BASED_ERR_UNSUPPORTED),
    (dict(scale=math.inf), _lib.BASED_ERR_INVALID_ARGUMENT),
    (dict(out=S_IN + 128), _lib.BASED_ERR_INVALID_ARGUMENT),  # out overlaps the state
    (dict(norm=S_IN + 1024), _lib.BASED_ERR_INVALID_ARGUMENT),  # state and norm overlap
])
def test_decode_step_rejects_bad_arguments(kw, status):
    assert call_decode(**kw) == status


def test_noalloc_entry_point_validates_on_the_host():
    """based_forward_noalloc takes based_forward's arguments and rejects bad ones before any HIP call."""
    lib = _lib.lib()
    assert lib.based_noalloc_scratch_bytes() == 32 << 20
    for kw, status in ((dict(q=0), _lib.BASED_ERR_INVALID_ARGUMENT), (dict(B=0), _lib.BASED_ERR_INVALID_ARGUMENT),
                       (dict(K=12), _lib.BASED_ERR_UNSUPPORTED), (dict(scale=math.inf), _lib.BASED_ERR_INVALID_ARGUMENT),
                       (dict(out=FAKE), _lib.BASED_ERR_INVALID_ARGUMENT)):
        a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, T=64, H=2, K=16, V=64, scale=math.nan, out=0x80000000, dt=0)
        a.update(kw)
        got = lib.based_forward_noalloc(a["q"], a["k"], a["v"], a["B"], a["T"], a["H"], a["K"], a["V"], a["scale"],
                                        a["out"], a["dt"], None)
        assert got == status, (kw, got)


def test_automatic_plans_fit_the_static_scratch():
    """The workspace of every automatic plan over a grid of shapes stays within the static scratch of
    based_forward_noalloc (the largest needs about 21 MiB)."""
    lib = _lib.lib()
    cap = lib.based_noalloc_scratch_bytes()
    worst = 0
    for K in (8, 16):
        for V in (64, 128, 256, 512):
            for B, H in ((1, 1), (1, 2), (1, 16), (2, 8), (4, 16), (8, 32), (16, 64)):
                for T in (64, 300, 1024, 4096, 16384, 65000, 131072, 1 << 20):
                    if T * H * V * 4 > 2 ** 31 - 1:
                        continue
                    worst = max(worst, lib.based_forward_workspace_bytes(B, T, H, K, V))
    assert 0 < worst <= cap
