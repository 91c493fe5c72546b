"""Pins of the oracle's pointwise chain against exact arithmetic and closed forms.

Chain definition: "C-05. Kernel Fusion 代价边界", section 3 (y = a_s*y + b_s,
ReLU on even stages).  Affine collapse and its fp32 error level: "AIGC 基本功｜
算子融合与 CUDA Graph-Fusion", section 4.1 (V1 vs V3).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from exact import exact_chain, f32_value
from conftest import load_golden


def normwise(y, ref):
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref)) / np.max(np.abs(ref)))


@pytest.mark.parametrize("K", [1, 2, 3, 4, 6, 8])
@pytest.mark.parametrize("relu", [True, False])
def test_chain_f64_matches_exact_rationals(K, relu):
    x, a, b = synth.chain_inputs(37, K, salt=K)
    y = oracle.chain_f64(x, a, b, relu)
    for i in range(x.size):
        ex = exact_chain(x[i], a, b, relu)
        assert abs(Fraction(float(y[i])) - ex) <= Fraction(1, 10**13) * (1 + abs(ex))


@pytest.mark.parametrize("K", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("relu", [True, False])
def test_chain_f32fma_is_one_rounding_per_stage(K, relu):
    """Bit-exact against exact arithmetic rounded to fp32 after each stage."""
    x, a, b = synth.chain_inputs(41, K, salt=100 + K)
    # include values near zero so ReLU and sign changes are exercised
    x[:5] = np.array([0.0, -0.0, 1e-30, -1e-30, 0.05], dtype=np.float32)
    y = oracle.chain_f32fma(x, a, b, relu)
    for i in range(x.size):
        ex = exact_chain(x[i], a, b, relu, round_each_stage=True)
        assert Fraction(float(y[i])) == ex, (i, float(y[i]), float(ex))


def test_relu_even_stage_indexing():
    """Stage 0 is even: with K = 1 and a = 1, b = 0 the chain is ReLU(x);
    with K = 2 the second (odd) stage must not clamp."""
    x = np.array([-2.0, -0.5, 0.0, 0.5, 2.0], dtype=np.float32)
    one = np.ones(1, np.float32)
    zero = np.zeros(1, np.float32)
    assert np.array_equal(oracle.chain_f64(x, one, zero, True), np.maximum(x, 0).astype(np.float64))
    assert np.array_equal(oracle.chain_f64(x, one, zero, False), x.astype(np.float64))
    # stage 0: y = x (then ReLU), stage 1: y = y - 1 (no ReLU) -> negative values survive
    a = np.array([1.0, 1.0], np.float32)
    b = np.array([0.0, -1.0], np.float32)
    y = oracle.chain_f64(x, a, b, True)
    assert np.array_equal(y, np.maximum(x, 0).astype(np.float64) - 1.0)
    assert (y < 0).any()


def test_relu_final_even_stage_is_nonnegative():
    x, a, b = synth.chain_inputs(4096, 5, salt=7)
    y = oracle.chain_f64(x, a, b, True)
    assert (y >= 0).all()
    y2 = oracle.chain_f64(x, a[:4], b[:4], True)
    assert (y2 < 0).any()


def _affine_closed(x, A, B, K):
    """h_K = A^K h_0 + B (A^K - 1) / (A - 1), exactly; limit K*B when A = 1."""
    Ak = A ** K
    Bk = B * K if A == 1 else B * (Ak - 1) / (A - 1)
    return Ak * x + Bk


def test_affine_collapse_closed_form_f64():
    n = 2048
    x, a, b = synth.affine_inputs(n)
    A, B = f32_value(a[0]), f32_value(b[0])
    y = oracle.chain_f64(x, a, b, relu_even=False)
    ref = np.array([float(_affine_closed(f32_value(v), A, B, 8)) for v in x])
    assert normwise(y, ref) <= 1e-13
    # the closed form's constants for the fp32 coefficients
    assert abs(float(A ** 8) - 1.082856623830647) < 1e-15
    assert abs(float(B * (A ** 8 - 1) / (A - 1)) - 0.08285670099696478) < 1e-15


def test_affine_collapse_unit_slope_limit():
    x = np.array([0.25, -3.0, 7.5], dtype=np.float32)
    a = np.ones(6, np.float32)
    b = np.full(6, 0.125, np.float32)
    y = oracle.chain_f64(x, a, b, relu_even=False)
    assert np.array_equal(y, x.astype(np.float64) + 6 * 0.125)


def test_fp32_chain_error_level_matches_pages():
    """The fp32 chain is within the pages' fp32 error level of the collapsed form."""
    g = load_golden("affine_chain_error.json")
    n = 1048576
    x, a, b = synth.affine_inputs(n)
    A, B = f32_value(a[0]), f32_value(b[0])
    Ak, Bk = float(A ** 8), float(B * (A ** 8 - 1) / (A - 1))
    ref = x.astype(np.float64) * Ak + Bk          # exact up to fp64 rounding
    err = normwise(oracle.chain_f32fma(x, a, b, relu_even=False), ref)
    page = {r["n"]: r["rel_err"] for r in g["rows"]}[n]
    assert 1e-8 <= err <= 2 * page, (err, page)
    assert normwise(oracle.chain_f64(x, a, b, relu_even=False), ref) <= 1e-13
