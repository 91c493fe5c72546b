"""Pins of the byte/launch ledgers against the values the pages print.

Plan table: "K4 讲解：fusion 的三笔账", section 1.  Chain and attention-score
ledgers: "AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.2 and the
appendix ledger [A].  Causal kept fractions: same page, section 3.5.
"""
from fractions import Fraction

import pytest

from oracle import ledger
from conftest import load_golden

MIB = 1024 ** 2
GIB = 1024 ** 3


def test_split_plan_table():
    g = load_golden("k4_split_plans.json")
    for row in g["plans"]:
        assert ledger.plan_bytes(g["M"], g["N"], g["K"], row["plan"], g["elem_bytes"]) == row["bytes"]
        assert ledger.plan_launches(row["plan"]) == row["launches"]


def test_plans_with_one_cut_move_equal_bytes():
    for plan in ([1, 3], [2, 2], [3, 1]):
        assert ledger.plan_bytes(4096, 4096, 4096, plan) == 201334784
    for plan in ([1, 1, 2], [1, 2, 1], [2, 1, 1]):
        assert ledger.plan_bytes(4096, 4096, 4096, plan) == 268443648


def test_compositions_enumerate_every_plan():
    g = load_golden("k4_split_plans.json")
    plans = ledger.compositions(4)
    assert len(plans) == g["n_plans_for_4_stages"]
    assert sorted(map(tuple, plans)) == sorted(
        [(1, 1, 1, 1), (1, 1, 2), (1, 2, 1), (2, 1, 1), (1, 3), (2, 2), (3, 1), (4,)])
    for n in range(1, 8):
        ps = ledger.compositions(n)
        assert len(ps) == 2 ** (n - 1) and len({tuple(p) for p in ps}) == len(ps)
        assert all(sum(p) == n for p in ps)


@pytest.mark.parametrize("plan", [[], [0, 4], [5], [1, 1, 1], [2, -1, 3]])
def test_bad_plans_rejected(plan):
    with pytest.raises(ValueError):
        ledger.plan_bytes(16, 16, 16, plan)


def test_decode_model_consistency():
    """Weak pin: the decode byte counts with the back-solved 448 GB/s and the
    printed 5 us launch reproduce the printed 97.5 / 80.8 us."""
    g = load_golden("k4_split_plans.json")["decode_model"]
    bw = g["implied_bandwidth_GBps"] * 1e9
    t_unf = ledger.plan_bytes(16, 4096, 4096, [1, 1, 1, 1]) / bw * 1e6 + 4 * g["launch_us"]
    t_fus = ledger.plan_bytes(16, 4096, 4096, [4]) / bw * 1e6 + 1 * g["launch_us"]
    assert round(t_unf, 1) == g["unfused_us"] or abs(t_unf - g["unfused_us"]) < 0.06
    assert abs(t_fus - g["fused_us"]) < 0.06
    assert ledger.plan_bytes(16, 4096, 4096, [1, 1, 1, 1]) == 34742272
    assert ledger.plan_bytes(16, 4096, 4096, [4]) == 33955840


def test_chain_ledger_and_ratio():
    g = load_golden("fusion_lab_ledger.json")["chain"]
    unf = ledger.chain_bytes(g["n"], g["K"], fused=False, elem_bytes=g["elem_bytes"])
    fus = ledger.chain_bytes(g["n"], g["K"], fused=True, elem_bytes=g["elem_bytes"])
    assert round(unf / MIB, 1) == g["unfused_MiB_1dp"]
    assert round(fus / MIB, 1) == g["fused_MiB_1dp"]
    assert unf == g["ratio"] * fus
    for K in (1, 2, 3, 4, 6, 8, 17):
        for n in (1, 1023, 16777216):
            assert ledger.chain_bytes(n, K, False) == K * ledger.chain_bytes(n, K, True) == K * 8 * n


def test_attention_score_ledger():
    g = load_golden("fusion_lab_ledger.json")["attention_score"]
    B, H, S, d, eb = g["B"], g["H"], g["S"], g["d"], g["elem_bytes"]
    score = B * H * S * S * eb
    assert round(B * S * d * eb / MIB, 1) == g["activation_MiB_1dp"]
    assert round(score / GIB, 3) == g["score_GiB_3dp"]
    assert score // (B * S * d * eb) == g["blowup"] == H * S // d
    BH = B * H
    # no skipping (tile = S): read once, write once
    assert round(ledger.softmax_bytes(BH, S, S, fused=True) / GIB, 3) == g["fused_GiB_3dp"]
    unf = ledger.softmax_bytes(BH, S, S, fused=False)
    stats = 4 * BH * S * 4
    mask = score
    assert round((unf - stats - mask) / GIB, 3) == g["unfused_five_steps_GiB_3dp"]
    assert round(mask / GIB, 3) == g["materialised_mask_GiB_3dp"]
    assert unf == 9667870720
    for row in g["blowup_curve_HSd"]:
        assert H * row["S"] / d == row["x"]


def test_causal_kept_fractions():
    g = load_golden("causal_kept_fraction.json")
    S = g["S"]
    f = ledger.causal_kept_fraction(S)
    assert f == Fraction(S + 1, 2 * S)
    assert round(float(f) * 100, 1) == g["exact_percent_1dp"]
    for row in g["blocks"]:
        T = row["tile"]
        fb = ledger.causal_block_fraction(S, T)
        nb = S // T
        assert fb == Fraction(nb + 1, 2 * nb)
        assert float(f"{float(fb) * 100:.1f}") == row["percent_1dp"]
        # row-wise tile loads read exactly the block-level element count
        assert ledger.softmax_elements_read(S, T) == T * T * nb * (nb + 1) // 2


def test_softmax_fused_bytes_with_skipping():
    BH, S = 128, 2048
    assert ledger.softmax_bytes(BH, S, 64, True) == 1627389952
    assert ledger.softmax_bytes(BH, S, 128, True) == 1644167168
    assert ledger.softmax_bytes(BH, S, 256, True) == 1677721600
    assert ledger.softmax_elements_read(S, 64) == 2162688
    # partial last tile
    assert ledger.softmax_elements_read(65, 64) == 64 * 64 + 65
