"""Worked examples in tests/golden/: inputs and exact outputs derived by hand from the page's definition
(page "Write a fast Based (Taylor linear attention) forward kernel", fields spec_md and contract_md; each
file carries its derivation). The pages print no numeric example of their own, so these are the fixed
points the oracle is held to: the exact route must reproduce every rational, the float routes must agree
to rounding.
"""
import glob
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import based_ref_chunked, based_ref_direct, based_ref_rational
from oracle.based_direct_c import based_ref_direct_c

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FILES = sorted(glob.glob(os.path.join(GOLDEN, "*.txt")))


def load(path):
    fields = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = line.split(":", 1)
        fields[key.strip()] = val.split()
    B, T, H, K, V = (int(x) for x in fields["shape"])
    scale = Fraction(fields["scale"][0])
    q = np.array([float(Fraction(x)) for x in fields["q"]]).reshape(B, T, H, K)
    k = np.array([float(Fraction(x)) for x in fields["k"]]).reshape(B, T, H, K)
    v = np.array([float(Fraction(x)) for x in fields["v"]]).reshape(B, T, H, V)
    o = [Fraction(x) for x in fields["o"]]
    assert len(o) == B * T * H * V
    return q, k, v, scale, o


def bf16_bits(x):
    """bf16 bit patterns of values that bf16 holds exactly (the fixtures' inputs)."""
    f = np.asarray(x, dtype=np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64))
    u = f.view(np.uint32)
    assert np.all(u & 0xFFFF == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def test_fixtures_present():
    assert len(FILES) >= 3


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(p) for p in FILES])
def test_oracle_reproduces_worked_example(path):
    q, k, v, scale, o = load(path)
    # scale values in the fixtures are exact in binary floating point (1, 1/2)
    assert Fraction(float(scale)) == scale
    exact = based_ref_rational(q, k, v, float(scale))
    got = [x for b in exact for t in b for h in t for x in h]
    assert got == o
    want = np.array([float(x) for x in o]).reshape(v.shape)
    T = q.shape[1]
    for route in (based_ref_direct(q, k, v, float(scale)),
                  based_ref_chunked(q, k, v, float(scale), chunk=1),
                  based_ref_chunked(q, k, v, float(scale), chunk=2),
                  based_ref_chunked(q, k, v, float(scale), chunk=T),
                  based_ref_direct_c(bf16_bits(q), bf16_bits(k), bf16_bits(v), float(scale))):
        np.testing.assert_allclose(route, want, rtol=1e-14, atol=1e-15)
    # the C route evaluates any chosen rows on their own
    rows = np.arange(T)[::-1]
    np.testing.assert_allclose(based_ref_direct_c(bf16_bits(q), bf16_bits(k), bf16_bits(v), float(scale), rows),
                               want[:, rows], rtol=1e-14, atol=1e-15)
