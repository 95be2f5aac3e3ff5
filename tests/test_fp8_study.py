"""CPU checks of the operand-precision study (oracle/fp8_study.py): the format rounding is right, the
emulation with no rounding is the page's chunked algorithm, and its conclusion on a small shape."""
import numpy as np
import pytest

from oracle import based_ref_chunked, bf16_to_f64, errors
from oracle.fp8_study import emulate_forward, round_to_format, study
from taylor_feature_map_amd.inputs import f32_to_bf16_bits, make_qkv


def test_e4m3_rounding_by_hand():
    # 4 significant bits: 1, 1.125, 1.25, ...; halfway cases go to the even significand.
    x = np.array([1.0625, 1.1875, 1.3, -2.7, 448.0, 500.0, 2.0 ** -9, 1.4 * 2.0 ** -9, 0.0])
    want = np.array([1.0, 1.25, 1.25, -2.75, 448.0, 448.0, 2.0 ** -9, 2.0 ** -9, 0.0])
    np.testing.assert_array_equal(round_to_format(x, "e4m3"), want)


def test_e5m2_rounding_by_hand():
    x = np.array([1.1, 1.125, 1.375, 3.3, 60000.0, 2.0 ** -16 * 1.6])
    want = np.array([1.0, 1.0, 1.5, 3.5, 57344.0, 2.0 ** -15])
    np.testing.assert_array_equal(round_to_format(x, "e5m2"), want)


def test_bf16_rounding_matches_the_input_generator():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(10000) * np.exp2(rng.integers(-20, 20, 10000))).astype(np.float32)
    np.testing.assert_array_equal(round_to_format(x.astype(np.float64), "bf16"), bf16_to_f64(f32_to_bf16_bits(x)))


def test_unrounded_emulation_is_the_chunked_algorithm():
    qb, kb, vb = make_qkv(1, 300, 2, 8, 16, seed=4)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    o = emulate_forward(q, k, v, None, 128, intra="f64", readout="f64", update="f64")
    np.testing.assert_allclose(o, based_ref_chunked(q, k, v, None, 128), rtol=0, atol=1e-12)


def test_study_conclusion_small():
    """bf16 operands (the kernels) pass the gate; fp8 (e4m3) operands fail it even with per-block scales."""
    rows = {name: (m, r) for name, m, r in study(T=512)}
    m, r = rows["bf16 everywhere (the kernels)"]
    assert m <= 2e-2 and r <= 5e-3
    for name in ("e4m3 intra only", "e4m3 everywhere", "e5m2 everywhere"):
        assert rows[name][1] > 5e-3, name
    # narrower ranges do not rescue it: finer scales, or fp8 on the quadratic feature block only
    for name in ("e4m3 intra only, 8-entry scales", "e4m3 read-out only, 8-entry scales",
                 "e4m3 read-out, quadratic features only", "e4m3 update, quadratic features only"):
        assert rows[name][1] > 5e-3, name
