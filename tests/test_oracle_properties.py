"""Randomised agreement of the oracle's three routes (CPU): the definition written out, the page's chunked
feature-map algorithm at any chunk length, and exact rationals. Page "Write a fast Based (Taylor linear
attention) forward kernel": field spec_md (the definition and phi(q).phi(k) = 1 + s + s^2/2, which makes
the chunked form an exact rearrangement) and field reference_src (the chunked algorithm).

Values are bf16-representable (so the rational route sees the same inputs exactly); scales are fp32.
"""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from oracle import based_ref_chunked, based_ref_direct, based_ref_rational, rational_to_f64  # noqa: E402
from oracle.based_direct_c import based_ref_direct_c  # noqa: E402


def _bf16(x):
    """Round float32 values to the nearest bf16 (ties to even) and return them as float64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


@st.composite
def problems(draw, max_t=40, max_k=6, max_v=5):
    B = draw(st.integers(1, 2))
    T = draw(st.integers(1, max_t))
    H = draw(st.integers(1, 2))
    K = draw(st.integers(1, max_k))
    V = draw(st.integers(1, max_v))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    spread = draw(st.sampled_from([0.25, 1.0, 3.0]))
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((B, T, H, K)) * spread)
    k = _bf16(rng.standard_normal((B, T, H, K)) * spread)
    v = _bf16(rng.standard_normal((B, T, H, V)))
    scale = draw(st.one_of(st.none(), st.floats(-2.0, 2.0, width=32)))
    return q, k, v, scale


@settings(max_examples=60, deadline=None)
@given(problems(), st.integers(1, 50))
def test_chunked_equals_direct_for_any_chunk(prob, chunk):
    q, k, v, scale = prob
    d = based_ref_direct(q, k, v, scale)
    c = based_ref_chunked(q, k, v, scale, chunk=chunk)
    np.testing.assert_allclose(c, d, rtol=1e-10, atol=1e-12)


@settings(max_examples=25, deadline=None)
@given(problems(max_t=6, max_k=3, max_v=2))
def test_float_routes_match_exact_rationals(prob):
    q, k, v, scale = prob
    exact = rational_to_f64(based_ref_rational(q, k, v, scale))
    np.testing.assert_allclose(based_ref_direct(q, k, v, scale), exact, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(based_ref_chunked(q, k, v, scale, chunk=2), exact, rtol=1e-12, atol=1e-14)


def _bits(x):
    """bf16 bit patterns of float64 values that are bf16 already."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@settings(max_examples=40, deadline=None)
@given(problems(max_t=300, max_k=16, max_v=70), st.data())
def test_c_definition_equals_numpy_definition(prob, data):
    """The plain-C route (the definition's loops, float64) and the numpy route agree to rounding, on all rows
    and on any chosen subset of rows."""
    q, k, v, scale = prob
    d = based_ref_direct(q, k, v, scale)
    c = based_ref_direct_c(_bits(q), _bits(k), _bits(v), scale)
    np.testing.assert_allclose(c, d, rtol=1e-11, atol=1e-13)
    T = q.shape[1]
    rows = np.array(data.draw(st.lists(st.integers(0, T - 1), min_size=1, max_size=8)), dtype=np.int64)
    cr = based_ref_direct_c(_bits(q), _bits(k), _bits(v), scale, rows)
    np.testing.assert_allclose(cr, d[:, rows], rtol=1e-11, atol=1e-13)


@settings(max_examples=20, deadline=None)
@given(problems(max_t=6, max_k=3, max_v=2))
def test_c_definition_matches_exact_rationals(prob):
    q, k, v, scale = prob
    exact = rational_to_f64(based_ref_rational(q, k, v, scale))
    np.testing.assert_allclose(based_ref_direct_c(_bits(q), _bits(k), _bits(v), scale), exact, rtol=1e-12,
                               atol=1e-14)
