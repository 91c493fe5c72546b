"""Pins of the causal attention oracle (plain definition of attention under the
causal mask of "AIGC 基本功", section 3.5, the result an online-softmax kernel
reaches without materialising the scores).  Each check compares the oracle
with something its own formula does not produce: closed forms (constant
values, prefix means), a constructed input whose answer is known, and
invariances that a dropped term, a wrong mask direction, an off-by-one or a
swapped operand would break."""
import numpy as np
import pytest

import oracle
import synth


def bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def val(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def test_constant_values_give_the_constant():
    """Softmax weights sum to one: if every key carries the same value vector
    c, every output row is c, whatever Q and K are."""
    Q, K, _ = synth.attention_inputs(2, 37, 16, salt=1)
    c = bf16(np.linspace(-3, 3, 16))
    V = np.broadcast_to(c, Q.shape).copy()
    O = oracle.causal_attention_f64(Q, K, V, 0.25)
    assert np.max(np.abs(O - val(c))) < 1e-13


@pytest.mark.parametrize("how", ["zero_q", "zero_scale"])
def test_uniform_weights_give_the_prefix_mean(how):
    """Equal scores (Q = 0, or scale = 0) weight the causal prefix uniformly:
    O_i = (1 / (i + 1)) sum_{j <= i} V_j, a running mean."""
    Q, K, V = synth.attention_inputs(3, 50, 8, salt=2)
    scale = 0.3
    if how == "zero_q":
        Q = np.zeros_like(Q)
    else:
        scale = 0.0
    O = oracle.causal_attention_f64(Q, K, V, scale)
    v = val(V)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, 51)[None, :, None]
    assert np.max(np.abs(O - prefix_mean)) < 1e-12


def test_first_row_is_its_own_value():
    Q, K, V = synth.attention_inputs(4, 9, 32, salt=3)
    O = oracle.causal_attention_f64(Q, K, V, 1.7)
    assert np.array_equal(O[:, 0, :], val(V[:, 0, :]))


def test_dominant_key_selects_its_value():
    """K_j = 30 e_j and Q_i = e_{floor(i/2)}: query i scores key floor(i/2)
    at 30 and every other key at 0, so O_i = V_{floor(i/2)} up to e^-30.
    Swapping the roles of Q and K, or reading the mask the wrong way, selects
    other rows."""
    S, D = 12, 16
    K = np.zeros((1, S, D), np.float32)
    Q = np.zeros((1, S, D), np.float32)
    for j in range(S):
        K[0, j, j] = 30.0
    for i in range(S):
        Q[0, i, i // 2] = 1.0
    _, _, V = synth.attention_inputs(1, S, D, salt=4)
    O = oracle.causal_attention_f64(bf16(Q), bf16(K), V, 1.0)
    want = val(V)[0, [i // 2 for i in range(S)], :]
    assert np.max(np.abs(O[0] - want)) < 1e-11


def test_causality_later_keys_do_not_matter_but_the_diagonal_does():
    Q, K, V = synth.attention_inputs(1, 40, 16, salt=5)
    O = oracle.causal_attention_f64(Q, K, V, 0.5)
    i = 17
    K2, V2 = K.copy(), V.copy()
    rng = np.random.default_rng(6)
    K2[0, i + 1:] = bf16(rng.standard_normal((40 - i - 1, 16)))
    V2[0, i + 1:] = bf16(rng.standard_normal((40 - i - 1, 16)))
    O2 = oracle.causal_attention_f64(Q, K2, V2, 0.5)
    assert np.array_equal(O[0, :i + 1], O2[0, :i + 1])
    assert not np.allclose(O[0, i + 1:], O2[0, i + 1:])
    V3 = V.copy()
    V3[0, i] = bf16(val(V[0, i]) + 1.0)           # key i is seen by query i
    O3 = oracle.causal_attention_f64(Q, K, V3, 0.5)
    assert not np.allclose(O[0, i], O3[0, i])
    assert np.array_equal(O[0, :i], O3[0, :i])


def test_shifting_every_key_by_one_vector_changes_nothing():
    """q.(k_j + c) = q.k_j + q.c: a per-row constant, which softmax removes."""
    Q, _, V = synth.attention_inputs(2, 33, 8, salt=7)
    # keys on a quarter-integer grid, so that the shifted keys are exact in bf16
    K = bf16(np.random.default_rng(11).integers(-8, 9, (2, 33, 8)) / 4.0)
    c = np.array([0.5, -1.0, 2.0, 0.25, 0.0, -0.75, 1.5, 1.0])
    K2 = bf16(val(K) + c)
    assert np.array_equal(val(K2), val(K) + c)
    O = oracle.causal_attention_f64(Q, K, V, 0.4)
    O2 = oracle.causal_attention_f64(Q, K2, V, 0.4)
    assert np.max(np.abs(O - O2)) < 1e-12


def test_last_row_ignores_key_order():
    Q, K, V = synth.attention_inputs(1, 30, 8, salt=8)
    perm = np.random.default_rng(9).permutation(30)
    O = oracle.causal_attention_rows(Q, K, V, 0.7, [29])
    Op = oracle.causal_attention_rows(Q, K[:, perm], V[:, perm], 0.7, [29])
    assert np.max(np.abs(O - Op)) < 1e-13


def test_rows_agree_with_all_rows():
    Q, K, V = synth.attention_inputs(2, 65, 128, salt=10)
    full = oracle.causal_attention_f64(Q, K, V, 128 ** -0.5).reshape(-1, 128)
    ids = np.array([0, 1, 63, 64, 65, 129])
    assert np.array_equal(oracle.causal_attention_rows(Q, K, V, 128 ** -0.5, ids), full[ids])


def test_two_keys_reduce_to_the_logistic_function():
    """Query 1 sees keys 0 and 1: O_1 = V_0 + sigma(d) (V_1 - V_0) with
    d = scale * q_1.(k_1 - k_0), sigma the logistic function."""
    from scipy.special import expit
    Q, K, V = synth.attention_inputs(3, 2, 16, salt=12)
    scale = 0.37
    O = oracle.causal_attention_f64(Q, K, V, scale)
    q, k, v = val(Q), val(K), val(V)
    d = scale * np.einsum("hd,hd->h", q[:, 1], k[:, 1] - k[:, 0])
    want = v[:, 0] + expit(d)[:, None] * (v[:, 1] - v[:, 0])
    assert np.max(np.abs(O[:, 1] - want)) < 1e-13


def test_single_rows_match_library_softmax_and_matmul():
    """Row i reduces to scipy's softmax of the scaled masked scores times V,
    with numpy's matmul for the products."""
    from scipy.special import softmax
    Q, K, V = synth.attention_inputs(2, 70, 128, salt=13)
    scale = 128 ** -0.5
    q, k, v = val(Q), val(K), val(V)
    rows = [(0, 0), (0, 1), (0, 31), (1, 64), (1, 69)]
    got = oracle.causal_attention_rows(Q, K, V, scale, [h * 70 + i for h, i in rows])
    for t, (h, i) in enumerate(rows):
        w = softmax(scale * (k[h, :i + 1] @ q[h, i]))
        assert np.max(np.abs(got[t] - w @ v[h, :i + 1])) < 1e-12
