"""Pins of the RMSNorm oracle (the row normalisation of the appendix ledger's
RMSNorm entry, "AIGC 基本功", section 3.2) and of its byte ledger: a library
norm, a closed form for constant rows, exact scale invariance, the unit root
mean square of the output, and the pages' printed MiB figures."""
import numpy as np

import oracle
from oracle import ledger
from conftest import load_golden

MIB = 1024 * 1024


def rows(r, d, salt):
    return np.random.default_rng(salt).standard_normal((r, d)).astype(np.float32)


def test_eps_zero_is_the_library_norm():
    """eps = 0: y = x * sqrt(d) / ||x||_2 * g, with numpy's norm."""
    x = rows(7, 96, 1)
    g = rows(1, 96, 2)[0]
    y = oracle.rmsnorm_f64(x, g, 0.0)
    x64 = x.astype(np.float64)
    want = x64 * np.sqrt(96.0) / np.linalg.norm(x64, axis=1, keepdims=True) * g.astype(np.float64)
    assert np.max(np.abs(y - want)) < 1e-13


def test_constant_rows_closed_form():
    """A row of c: mean square c^2, so y_j = c / sqrt(c^2 + eps) * g_j."""
    c = np.array([[2.0], [-0.5], [0.0]], np.float32)
    x = np.repeat(c, 33, axis=1)
    g = np.linspace(-1, 1, 33).astype(np.float32)
    eps = 1e-5
    y = oracle.rmsnorm_f64(x, g, eps)
    want = c.astype(np.float64) / np.sqrt(c.astype(np.float64) ** 2 + eps) * g.astype(np.float64)
    assert np.max(np.abs(y - want)) < 1e-15


def test_power_of_two_scaling_is_exact_without_eps():
    """Scaling a row by 2 scales its mean square by exactly 4 and the root by
    exactly 2, so with eps = 0 the output is bit-identical."""
    x = rows(5, 64, 3)
    g = rows(1, 64, 4)[0]
    assert np.array_equal(oracle.rmsnorm_f64(x, g, 0.0), oracle.rmsnorm_f64(2 * x, g, 0.0))


def test_unit_gain_gives_unit_root_mean_square():
    x = rows(9, 4096, 5)
    y = oracle.rmsnorm_f64(x, np.ones(4096, np.float32), 0.0)
    assert np.max(np.abs(np.mean(y * y, axis=1) - 1.0)) < 1e-12


def test_eps_enters_under_the_root():
    """Doubling eps on a row of tiny values moves y exactly as the closed form
    says: a dropped or misplaced eps shows here."""
    x = np.full((1, 10), 1e-3, np.float32)
    g = np.ones(10, np.float32)
    for eps in (1e-6, 2e-6):
        y = oracle.rmsnorm_f64(x, g, eps)
        xv = float(np.float32(1e-3))
        assert abs(y[0, 0] - xv / np.sqrt(xv * xv + eps)) < 1e-15


def test_pages_rmsnorm_ledger():
    g = load_golden("fusion_lab_ledger.json")["rmsnorm"]
    n, b = g["n"], g["elem_bytes"]
    unf = ledger.rmsnorm_bytes(n, False, b)
    fus = ledger.rmsnorm_bytes(n, True, b)
    assert f"{unf / MIB:.1f}" == f"{g['unfused_MiB_1dp']:.1f}"
    assert f"{fus / MIB:.1f}" == f"{g['fused_MiB_1dp']:.1f}"
    assert unf // fus == g["ratio"]
