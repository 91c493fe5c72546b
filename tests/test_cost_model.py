"""The split-plan time model ("K4 讲解", section 2) against the figures the page
prints: with the page's stated launch cost and register rule, and the
bandwidth and compute rate its figures imply, the model reproduces the decode
plans' 80.8 / 97.5 us, the 4096^3 plan's ~3.45 ms and the register-heavy
example's ~1.21 / ~1.81 ms, and picks the page's best plans."""
import gemm_epilogues_amd as fc
from conftest import load_golden

G = load_golden("k4_cost_model.json")


def pages_model():
    st, im = G["model_stated"], G["model_implied"]
    return fc.cost_model(im["hbm_GBps"] * 1e9, im["flops_TFLOPs"] * 1e12, st["launch_us"] * 1e-6,
                         levels=((st["reg_limit"], 1.0),), spill_factor=st["spill_penalty"])


def test_decode_shape_figures():
    m = pages_model()
    st = fc.fc_gemm_epilogue_stages(16, 4096, 4096)
    t4 = fc.fc_segments_time(st, [4], 2, m) * 1e6
    t1111 = fc.fc_segments_time(st, [1, 1, 1, 1], 2, m) * 1e6
    g = G["decode_16x4096x4096"]
    assert f"{t4:.1f}" == f"{g['plan4_us_1dp']:.1f}"
    assert f"{t1111:.1f}" == f"{g['plan1111_us_1dp']:.1f}"
    # the printed saving is the difference of the two printed (1-decimal) figures
    assert abs((round(t1111, 1) - round(t4, 1)) - g["saving_us_1dp"]) < 1e-9
    # three launches of 5 us are most of the saving
    assert 3 * G["model_stated"]["launch_us"] == g["launch_share_us"]
    assert fc.fc_best_split(st, 2, m)[0] == g["best"]


def test_square_shape_figure_and_best_plan():
    m = pages_model()
    st = fc.fc_gemm_epilogue_stages(4096, 4096, 4096)
    t4 = fc.fc_segments_time(st, [4], 2, m) * 1e3
    assert abs(t4 - G["square_4096"]["plan4_ms_approx"]) < 0.01
    assert fc.fc_best_split(st, 2, m)[0] == G["square_4096"]["best"]


def test_register_heavy_example():
    m = pages_model()
    h = G["heavy"]
    st = [(s["writes"], s["ext_reads"], s["flops"], s["live_regs"]) for s in h["stages"]]
    t11 = fc.fc_segments_time(st, [1, 1], h["elem_bytes"], m) * 1e3
    t2 = fc.fc_segments_time(st, [2], h["elem_bytes"], m) * 1e3
    assert abs(t11 - h["plan11_ms_approx"]) < 0.005
    assert abs(t2 - h["plan2_ms_approx"]) < 0.01
    assert fc.fc_best_split(st, h["elem_bytes"], m)[0] == h["best"]


def test_segment_bytes_match_the_plan_ledger():
    """With unit bandwidth, no compute, no launch and no register factor, the
    estimate is the plan's byte count."""
    m = fc.cost_model(1.0, 1e300, 0.0, levels=((1 << 30, 1.0),))
    for M, N, K in [(16, 4096, 4096), (4096, 4096, 4096), (300, 1000, 72)]:
        st = fc.fc_gemm_epilogue_stages(M, N, K)
        for plan in ([4], [1, 3], [2, 2], [3, 1], [1, 1, 2], [1, 1, 1, 1]):
            assert fc.fc_segments_time(st, plan, 2, m) == fc.fc_plan_bytes(M, N, K, plan)


def test_register_peaks_of_the_pages_table():
    """Fused segments sum their stages' live registers: 128 / 128 / 136 / 160
    for the four plans of the page's table (the factor steps at the level)."""
    st = fc.fc_gemm_epilogue_stages(64, 64, 64)
    regs = [s.live_regs for s in st]
    peaks = {(1, 1, 1, 1): 128, (1, 3): 128, (2, 2): 136, (4,): 160}
    for plan, peak in peaks.items():
        seg, s0 = [], 0
        for p in plan:
            seg.append(sum(regs[s0:s0 + p]))
            s0 += p
        assert max(seg) == peak
    # a level at 159 puts only the fully fused plan past it
    m = fc.cost_model(1e12, 1e300, 0.0, levels=((159, 1.0),), spill_factor=2.0)
    base = fc.cost_model(1e12, 1e300, 0.0, levels=((1 << 30, 1.0),))
    for plan in ([1, 3], [2, 2], [1, 1, 1, 1]):
        assert fc.fc_segments_time(st, plan, 2, m) == fc.fc_segments_time(st, plan, 2, base)
    assert fc.fc_segments_time(st, [4], 2, m) == 2 * fc.fc_segments_time(st, [4], 2, base)


def test_invalid_arguments():
    m = fc.cost_model(1e12, 1e12, 1e-6)
    st = fc.fc_gemm_epilogue_stages(8, 8, 8)
    assert fc.fc_segments_time(st, [1, 2], 2, m) == -1.0
    assert fc.fc_segments_time(st, [0, 4], 2, m) == -1.0
    bad = fc.cost_model(0.0, 1e12, 1e-6)
    assert fc.fc_segments_time(st, [4], 2, bad) == -1.0
