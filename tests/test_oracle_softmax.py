"""Pins of the oracle's causal scaled softmax.

Definition: "AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.5 (query i
sees keys j <= i) and the appendix attention-tail section (max, subtract,
exp, sum, divide).  Pinned against scipy's softmax on the kept prefix, exact
special rows and invariances.
"""
import numpy as np
import pytest
from scipy.special import softmax as sp_softmax, expit

import oracle
import synth
from exact import bf16_bits_value

SCALE = float(np.float32(1.0 / np.sqrt(128.0)))


@pytest.mark.parametrize("S", [1, 2, 3, 17, 64, 65])
def test_softmax_vs_scipy_on_kept_prefix(S):
    s = synth.softmax_inputs(2, S, salt=S)
    out = oracle.causal_softmax_f64(s, SCALE)
    z = synth.bf16_bits_to_f32(s).astype(np.float64) * SCALE
    for bh in range(2):
        for i in range(S):
            ref = sp_softmax(z[bh, i, :i + 1])
            assert np.max(np.abs(out[bh, i, :i + 1] - ref)) <= 1e-14
            assert np.all(out[bh, i, i + 1:] == 0.0)
            assert np.all(out[bh, i, :i + 1] > 0.0)
            assert abs(out[bh, i].sum() - 1.0) <= 1e-13


def test_decode_of_bf16_bits_is_exact():
    s = synth.softmax_inputs(1, 8, salt=1).ravel()
    for h in s[:64]:
        assert oracle.bf16_to_double(int(h)) == float(bf16_bits_value(int(h)))


def test_row_zero_and_equal_scores():
    S = 33
    s = np.full((1, S, S), synth.f32_to_bf16_bits(np.float32(1.5)), dtype=np.uint16)
    out = oracle.causal_softmax_f64(s, SCALE)
    assert out[0, 0, 0] == 1.0 and np.all(out[0, 0, 1:] == 0.0)
    for i in range(S):
        assert np.allclose(out[0, i, :i + 1], 1.0 / (i + 1), rtol=0, atol=1e-15)


def test_two_key_row_is_logistic():
    """Row 1 keeps two keys: out_1 = 1 / (1 + exp(-(z_1 - z_0)))."""
    S = 2
    vals = np.array([[0.0, 0.0], [-1.5, 2.25]], dtype=np.float32)
    s = synth.f32_to_bf16_bits(vals).reshape(1, S, S)
    out = oracle.causal_softmax_f64(s, 0.5)
    d = 0.5 * (2.25 - (-1.5))
    assert abs(out[0, 1, 1] - expit(d)) <= 1e-15
    assert abs(out[0, 1, 0] - expit(-d)) <= 1e-15


def test_shift_and_scale_invariance():
    S = 40
    s = synth.softmax_inputs(1, S, salt=5)
    f = synth.bf16_bits_to_f32(s).astype(np.float64)
    # doubling is exact in bf16; halving the scale must give the same result
    s2 = synth.f32_to_bf16_bits((2.0 * f).astype(np.float32))
    a = oracle.causal_softmax_f64(s, SCALE)
    b = oracle.causal_softmax_f64(s2, SCALE / 2)
    assert np.max(np.abs(a - b)) <= 1e-15
    # adding a constant: small integers shifted by 4 stay exact in bf16
    ints = synth.rng("misc", 7).integers(-3, 4, (1, S, S)).astype(np.float32)
    c = oracle.causal_softmax_f64(synth.f32_to_bf16_bits(ints).reshape(1, S, S), 1.0)
    d = oracle.causal_softmax_f64(synth.f32_to_bf16_bits(ints + 4.0).reshape(1, S, S), 1.0)
    assert np.max(np.abs(c - d)) <= 1e-15
    assert np.max(np.abs(c[0, S - 1] - sp_softmax(ints[0, S - 1].astype(np.float64)))) <= 1e-15


def test_rows_api_matches_full():
    BH, S = 3, 20
    s = synth.softmax_inputs(BH, S, salt=2)
    full = oracle.causal_softmax_f64(s, SCALE).reshape(BH * S, S)
    rows = np.array([0, 19, 20, 59, 33])
    assert np.array_equal(oracle.causal_softmax_rows(s, SCALE, rows), full[rows])


def test_mask01_is_lower_triangle():
    m = oracle.causal_mask01(5)
    assert np.array_equal(m, np.tril(np.ones((5, 5))))
