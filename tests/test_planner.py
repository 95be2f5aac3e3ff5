"""CPU checks of the work plan (`based_forward_plan`, host code, no GPU): for any shape the segments are
whole chunks that cover the sequence exactly, segments shorter than 256 tokens come at most eight at a time,
the state pass splits segments in two exactly where its rule says, and the shapes whose plans were chosen by
measurement keep them."""
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import assume, given, settings, strategies as st  # noqa: E402

from taylor_feature_map_amd import plan  # noqa: E402


def slot_floats(K, cols):
    # 4-byte words of one segment sum: per feature tile, the value tiles' 64 lanes x 4 rows in bf16 (half a
    # word each; fp32 for K = 16 with 128 columns), plus the ones tile's 16 in fp32 (10 tiles for K = 16, 3
    # for K = 8)
    per_entry = 1.0 if (K == 16 and cols == 128) else 0.5
    return (10 if K == 16 else 3) * (int((cols // 16) * 4 * 64 * per_entry) + 16)


def chunk(K, cols):
    return 128 if (K == 16 and cols == 128) else 64


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 16), st.integers(1, 200000), st.integers(1, 64), st.sampled_from([8, 16]),
       st.sampled_from([64, 128, 192, 256, 512]))
def test_plan_invariants(B, T, H, K, V):
    assume(T * H * V * 4 <= 2 ** 31 - 1)  # the library's 32-bit row ranges
    G, L, ws = plan(B, T, H, K, V)
    assert L % 64 == 0 and L >= 64
    assert G == -(-T // L) and (G - 1) * L < T <= G * L
    assert G <= 8 or L >= 256, "more than eight segments shorter than 256 tokens"
    assert (ws == 0) == (G == 1)
    if G > 1:
        # the workspace holds `sub` sums per (b, h, item, segment but the last): it tells the item width and
        # the number of pieces the state pass sums each segment in
        found = [(c, sub) for c in ((128, 64) if V % 128 == 0 else (64,)) for sub in (1, 2)
                 if ws == B * H * (V // c) * (G - 1) * sub * slot_floats(K, c) * 4]
        assert len(found) == 1, (ws, found)
        width, sub = found[0]
        C = chunk(K, width)
        assert L % C == 0 and L >= (2 if K == 16 else 1) * C
        if K == 8 or V % 128 != 0:
            assert width == (128 if V % 128 == 0 else 64)
        assert sub == (2 if split_pieces(B, H, V, width, G, L) else 1)


def split_pieces(B, H, V, width, G, L):
    # two pieces per segment when the state pass would have at most one workgroup per CU (256) and the
    # pieces stay whole 64-token chunks of at least 1024 tokens
    state_items = B * H * (V // width) * (width // 64) * (G - 1)
    return state_items <= 256 and L % 128 == 0 and L // 2 >= 1024


@pytest.mark.parametrize("shape,seg,sub", [
    ((4, 16384, 32, 8, 128), 0, 2),      # 128 (b, h) pairs x 2 halves x 1 segment: two pieces (5% faster)
    ((4, 8192, 16, 16, 64), 0, 1),       # 448 state workgroups already
    ((8, 4096, 16, 16, 128), 2048, 2),   # forced two segments of 128-column items: 256 state workgroups
    ((8, 4096, 16, 16, 128), 1024, 1),   # pieces of 512 tokens: too short
    ((1, 65000, 16, 16, 64), 0, 1),
])
def test_state_pieces(shape, seg, sub):
    B, T, H, K, V = shape
    G, L, ws = plan(*shape, seg)
    width = 128 if (V % 128 == 0 and ws == B * H * (V // 128) * (G - 1) * sub * slot_floats(K, 128) * 4) else 64
    assert ws == B * H * (V // width) * (G - 1) * sub * slot_floats(K, width) * 4, (G, L, ws)


@pytest.mark.parametrize("shape,G,L", [
    ((1, 512, 2, 8, 64), 8, 64),          # short K = 8 sequence: one chunk per segment
    ((2, 512, 8, 16, 64), 4, 128),        # short K = 16 sequence: two chunks per segment
    ((1, 256, 4, 16, 128), 1, 256),       # two 128-token chunks: one kernel
    ((1, 4096, 16, 8, 128), 16, 256),     # at most eight segments shorter than 256 tokens
    ((1, 1024, 8, 8, 64), 8, 128),        # ... and then eight of the shortest length (18% faster than 4 x 256)
    ((1, 1536, 4, 8, 128), 8, 192),       # (9% faster than 6 x 256)
    ((2, 2048, 8, 16, 64), 8, 256),
    ((4, 8192, 16, 16, 64), 8, 1024),     # two waves per SIMD
    ((4, 8192, 16, 8, 64), 16, 512),      # K = 8 with 64 columns: two waves per SIMD as well
    ((4, 16384, 32, 8, 128), 2, 8192),    # K = 8 with 128 columns: one wave per SIMD
    ((1, 32768, 32, 8, 128), 8, 4096),
    ((8, 16384, 32, 16, 64), 1, 16384),   # the items alone fill every CU: no state pass
    ((8, 16384, 32, 8, 128), 1, 16384),
    ((16, 2048, 16, 16, 64), 1, 2048),
    ((8, 4096, 16, 16, 128), 1, 4096),    # 64-column items fill every CU where 128-column ones would not
    ((1, 2048, 16, 16, 128), 8, 256),     # short sequence: 64-column items (all CUs) over 128-column (half)
    ((8, 8192, 32, 16, 128), 1, 8192),    # 128-column items already fill every CU
    ((2, 16384, 32, 16, 128), 4, 4096),   # too few for either: 128-column items, 4 segments
    ((1, 65000, 16, 16, 64), 32, 2048),   # long sequence: scanned segment sums
])
def test_measured_plans(shape, G, L):
    assert plan(*shape)[:2] == (G, L)


def test_forced_segment_length_rounds_to_chunks():
    assert plan(1, 1000, 2, 16, 64, 100)[:2] == (8, 128)
    assert plan(1, 1000, 2, 16, 128, 100)[:2] == (8, 128)
    assert plan(1, 1000, 2, 16, 64, 5000)[:2] == (1, 1024)


def test_too_many_work_items_rejected():
    """The kernels number their work items in 32 bits: a shape with 2^30 (b, h) pairs is refused on the
    host (status 2, unsupported) instead of launching an oversized grid."""
    from taylor_feature_map_amd import _lib
    with pytest.raises(_lib.BasedError) as e:
        plan(1 << 20, 64, 1 << 10, 16, 64)
    assert e.value.status == _lib.BASED_ERR_UNSUPPORTED
    assert plan(1 << 12, 64, 1 << 10, 16, 64)[0] == 1  # 2^22 pairs, one segment: fine
