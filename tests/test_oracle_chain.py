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
from exact import exact_chain, f32_rne, f32_value
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


# ---------------------------------------------------------------- fat-probe sink
# The sink of the fat row ("C-05", section 3, API table) as read here: vector q
# of four elements belongs to lane q mod L; per element t_j = t_{j-1}/2 +
# y_{floor(jK/T)} (y_s the chain value after stage s), the element's term is
# sum_j t_j, and a lane adds its vectors' terms per component.


def _fat_sink_exact(x, a, b, relu, T, lanes, round_each=False):
    """Exact rational sink written from the definition (independent of the C
    code): optionally every step rounded to fp32, in the probe's order."""
    K = len(a)
    nvec = len(x) // 4
    out = [Fraction(0)] * (4 * lanes)
    rnd = f32_rne if round_each else (lambda v: v)
    for lane in range(lanes):
        for c in range(4):
            acc = Fraction(0)
            for q in range(lane, nvec, lanes):
                ys = []
                y = f32_value(x[4 * q + c])
                for s in range(K):
                    y = rnd(f32_value(a[s]) * y + f32_value(b[s]))
                    if relu and s % 2 == 0 and y < 0:
                        y = Fraction(0)
                    ys.append(y)
                ts, t = [], Fraction(0)
                for j in range(T):
                    t = rnd(t / 2 + ys[(j * K) // T])
                    ts.append(t)
                if T:
                    r = ts[-1]
                    for j in range(T - 2, -1, -1):
                        r = rnd(ts[j] + r)
                    acc = rnd(acc + r)
            out[4 * lane + c] = acc
    return out


def test_fat_sink_identity_chain_closed_form():
    """a = 1, b = 0: every y_s is ReLU(x), t_j = 2y(1 - 2^-(j+1)) and the
    element's term is 2y(T - 1 + 2^-T).  x in {-1, 0, 1}: every value is exact
    in fp32 at T = 16, so both evaluations equal the closed form bit for bit."""
    rng = np.random.default_rng(5)
    n, lanes, T, K = 4 * 37 + 3, 9, 16, 4
    x = rng.integers(-1, 2, n).astype(np.float32)
    a, b = np.ones(K, np.float32), np.zeros(K, np.float32)
    term = 2.0 * (T - 1 + 2.0 ** -T)
    expect = np.zeros(4 * lanes)
    for q in range(n // 4):
        expect[4 * (q % lanes): 4 * (q % lanes) + 4] += np.maximum(x[4 * q: 4 * q + 4], 0) * term
    assert np.array_equal(oracle.chain_fat_sink_f64(x, a, b, True, T, lanes), expect)
    assert np.array_equal(oracle.chain_fat_sink_f32(x, a, b, True, T, lanes).astype(np.float64), expect)
    # without ReLU the negative elements count with their sign
    expect_lin = np.zeros(4 * lanes)
    for q in range(n // 4):
        expect_lin[4 * (q % lanes): 4 * (q % lanes) + 4] += x[4 * q: 4 * q + 4] * term
    assert np.array_equal(oracle.chain_fat_sink_f64(x, a, b, False, T, lanes), expect_lin)


@pytest.mark.parametrize("K,T", [(4, 16), (4, 48), (3, 16), (8, 48), (4, 128)])
def test_fat_sink_stage_mapping_closed_form(K, T):
    """x = 0, a = 1, b_s distinct, no ReLU: y_s = b_0 + ... + b_s, and
    sum_j t_j = sum_i y_{s(i)} * 2 (1 - 2^(i-T)) (a geometric sum in place of the
    recurrence), which fixes which stage feeds which temporary."""
    b = (np.arange(1, K + 1, dtype=np.float32) * np.float32(0.125)) ** 2
    a = np.ones(K, np.float32)
    x = np.zeros(4, np.float32)
    ys = np.cumsum([Fraction(float(v)) for v in b])
    total = sum(ys[(i * K) // T] * 2 * (1 - Fraction(2) ** (i - T)) for i in range(T))
    got = oracle.chain_fat_sink_f64(x, a, b, False, T, 1)
    assert np.all(np.abs(got - float(total)) <= 1e-13 * float(total))
    got32 = oracle.chain_fat_sink_f32(x, a, b, False, T, 1).astype(np.float64)
    assert np.all(np.abs(got32 - float(total)) <= 4 * T * 2.0 ** -24 * float(total))


@pytest.mark.parametrize("K,T,relu,n,lanes", [(1, 16, True, 20, 2), (2, 16, True, 37, 3), (3, 16, False, 29, 1),
                                              (4, 48, True, 40, 4), (4, 16, True, 13, 5)])
def test_fat_sink_exact_rationals(K, T, relu, n, lanes):
    """Against exact arithmetic: the fp64 sink within 1e-12 of the exact value
    (relative to the sum of |t_j|); the fp32 sink bit for bit equal to exact
    arithmetic rounded to fp32 after every step in the probe's order."""
    x, a, b = synth.chain_inputs(n, K, salt=300 + 10 * K + T)
    ex = _fat_sink_exact(x, a, b, relu, T, lanes)
    got, absd = oracle.chain_fat_sink_f64(x, a, b, relu, T, lanes, with_abs=True)
    for g, e, s in zip(got, ex, absd):
        assert abs(Fraction(float(g)) - e) <= Fraction(1, 10**12) * (Fraction(float(s)) + 1)
    ex32 = _fat_sink_exact(x, a, b, relu, T, lanes, round_each=True)
    got32 = oracle.chain_fat_sink_f32(x, a, b, relu, T, lanes)
    for g, e in zip(got32, ex32):
        assert Fraction(float(g)) == e


def test_fat_sink_lane_geometry_and_tail():
    """One nonzero vector q lands in lane q mod L only; elements past the last
    whole vector never reach the sink; T = 0 leaves the sink zero."""
    K, T, lanes = 2, 16, 7
    a, b = np.ones(K, np.float32), np.zeros(K, np.float32)
    n = 4 * 50 + 3
    for q in (0, 6, 7, 23, 49):
        x = np.zeros(n, np.float32)
        x[4 * q + 2] = 1.0
        s = oracle.chain_fat_sink_f64(x, a, b, True, T, lanes)
        nz = np.flatnonzero(s)
        assert list(nz) == [4 * (q % lanes) + 2], (q, nz)
    x = np.zeros(n, np.float32)
    x[-3:] = 5.0
    assert not oracle.chain_fat_sink_f64(x, a, b, True, T, lanes).any()
    x, a2, b2 = synth.chain_inputs(n, K, salt=3)
    assert not oracle.chain_fat_sink_f64(x, a2, b2, True, 0, lanes).any()
    assert not oracle.chain_fat_sink_f32(x, a2, b2, True, 0, lanes).any()


def test_fat_sink_f32_tracks_f64():
    """At the probe's own geometry (2048 workgroups x 256 lanes, K = 4, T = 48)
    on 1M elements: the fp32 sink is within 64 u of the fp64 one relative to
    the sum of |t_j| (T + K + the lane's vectors roundings, each at most u of
    that scale)."""
    n, K, T, lanes = 1 << 20, 4, 48, 2048 * 256
    x, a, b = synth.chain_inputs(n, K, salt=77)
    s64, absd = oracle.chain_fat_sink_f64(x, a, b, True, T, lanes, with_abs=True)
    s32 = oracle.chain_fat_sink_f32(x, a, b, True, T, lanes).astype(np.float64)
    assert np.all(np.abs(s32 - s64) <= 64 * 2.0 ** -24 * absd + 1e-30)
