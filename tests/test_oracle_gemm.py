"""Pins of the oracle's GEMM + bias + GELU + residual chain.

Chain: "K4 讲解：fusion 的三笔账", section 1 (mm -> bias -> gelu -> res).  GELU
in erf form, z * Phi(z), pinned against textbook normal-CDF values.  The GEMM
is pinned against exact rational brute force, integer matmul and numpy's fp64
matmul.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from exact import f16_bits_value
from conftest import load_golden


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (8, 7, 6), (17, 5, 33), (3, 33, 17)])
def test_gemm_exact_rationals(M, N, K):
    A, B, _, _ = synth.gemm_inputs(M, N, K, salt=M * 100 + N * 10 + K)
    C = oracle.gemm_f64(A, B)
    Av = [[f16_bits_value(A[i, k]) for k in range(K)] for i in range(M)]
    Bv = [[f16_bits_value(B[k, j]) for j in range(N)] for k in range(K)]
    for i in range(M):
        for j in range(N):
            ex = sum((Av[i][k] * Bv[k][j] for k in range(K)), Fraction(0))
            assert abs(Fraction(float(C[i, j])) - ex) <= Fraction(1, 10**14) * (1 + abs(ex))


def test_gemm_integer_exact():
    M, N, K = 19, 40, 300
    A, B = synth.gemm_int_inputs(M, N, K)
    Ai = A.view(np.float16).astype(np.int64)
    Bi = B.view(np.float16).astype(np.int64)
    C = oracle.gemm_f64(A, B)
    assert np.array_equal(C, (Ai @ Bi).astype(np.float64))


def test_gemm_vs_numpy_matmul():
    M, N, K = 48, 80, 256
    A, B, _, _ = synth.gemm_inputs(M, N, K)
    Af = A.view(np.float16).astype(np.float64)
    Bf = B.view(np.float16).astype(np.float64)
    C = oracle.gemm_f64(A, B)
    ref = Af @ Bf
    assert np.max(np.abs(C - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_gelu_normal_cdf_table():
    g = load_golden("normal_cdf_table.json")
    for row in g["rows"]:
        z = row["z"]
        got = oracle.gelu(z)
        assert abs(got - z * row["phi"]) <= abs(z) * 0.6e-4 + 1e-15, (z, got)


def test_gelu_special_values():
    assert oracle.gelu(0.0) == 0.0
    for z in (0.1, 0.7, 1.3, 2.9, 5.0):
        # erf is odd, so GELU(-z) = GELU(z) - z
        assert abs(oracle.gelu(-z) - (oracle.gelu(z) - z)) <= 1e-15 * (1 + z)
    assert abs(oracle.gelu(12.0) - 12.0) <= 1e-15 * 12
    assert -1e-20 < oracle.gelu(-12.0) <= 0.0
    # monotone above the minimum near z = -0.75
    zs = np.linspace(-0.7, 6, 200)
    v = [oracle.gelu(z) for z in zs]
    assert all(b > a for a, b in zip(v, v[1:]))


def test_epilogue_residual_indexing():
    """A = 0 and bias = 0 give Y = GELU(0) + R = R exactly; a transposed
    or shifted residual would fail on this non-square shape."""
    M, N, K = 5, 11, 8
    _, _, _, R = synth.gemm_inputs(M, N, K, salt=3)
    A = np.zeros((M, K), np.uint16)
    B = synth.gemm_inputs(M, N, K, salt=4)[1]
    bias = np.zeros(N, np.uint16)
    Y = oracle.gemm_epilogue_f64(A, B, bias, R)
    assert np.array_equal(Y, R.view(np.float16).astype(np.float64))


def test_epilogue_bias_broadcast_and_gelu():
    """A = 0, R = 0: Y[i, j] = GELU(bias[j]) = bias[j] * Phi(bias[j])."""
    g = load_golden("normal_cdf_table.json")
    zs = [r["z"] for r in g["rows"]]
    phis = [r["phi"] for r in g["rows"]]
    N = len(zs)
    M, K = 3, 4
    bias = synth.f64_to_f16_bits(np.array(zs))    # table points are exact in fp16
    A = np.zeros((M, K), np.uint16)
    B = np.zeros((K, N), np.uint16)
    R = np.zeros((M, N), np.uint16)
    Y = oracle.gemm_epilogue_f64(A, B, bias, R)
    for j in range(N):
        assert np.all(Y[:, j] == Y[0, j])
        assert abs(Y[0, j] - zs[j] * phis[j]) <= abs(zs[j]) * 0.6e-4 + 1e-15


def test_epilogue_sampled_matches_full():
    M, N, K = 9, 24, 40
    A, B, bias, R = synth.gemm_inputs(M, N, K, salt=9)
    Y = oracle.gemm_epilogue_f64(A, B, bias, R)
    rows = np.array([0, 8, 4, 3, 8])
    cols = np.array([0, 23, 11, 5, 0])
    assert np.array_equal(oracle.gemm_epilogue_at(A, B, bias, R, rows, cols), Y[rows, cols])


def test_epilogue_large_positive_preactivation_passes_through():
    """For a large pre-activation GELU is the identity: Y = A.B + bias + R."""
    M, N, K = 4, 6, 16
    A = synth.f64_to_f16_bits(np.full((M, K), 0.5))
    B = synth.f64_to_f16_bits(np.full((K, N), 1.5))          # A.B = 12
    bias = synth.f64_to_f16_bits(np.arange(N) * 0.25)
    R = synth.f64_to_f16_bits(np.arange(M * N).reshape(M, N) * 0.125)
    Y = oracle.gemm_epilogue_f64(A, B, bias, R)
    ref = 12.0 + (np.arange(N) * 0.25)[None, :] + np.arange(M * N).reshape(M, N) * 0.125
    assert np.max(np.abs(Y - ref)) <= 1e-12


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (17, 40, 24), (64, 128, 256), (130, 72, 520)])
def test_matmul_form_equals_plain_form(M, N, K):
    """The form that takes the product step from numpy's fp64 matmul (used at
    4096^3, where the plain triple loop takes minutes) gives the plain
    oracle's Y to fp64 rounding: the same bias, GELU and residual stages on a
    product formed by a different routine."""
    A, B, bias, R = synth.gemm_inputs(M, N, K, salt=400 + M)
    plain = oracle.gemm_epilogue_f64(A, B, bias, R)
    fast = oracle.gemm_epilogue_f64_matmul(A, B, bias, R)
    assert np.max(np.abs(fast - plain) / (1 + np.abs(plain))) <= 1e-12
