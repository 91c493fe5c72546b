"""GPU parity of the causal scaled-masked softmax (fused with block skipping,
and the unfused five-step baseline) against the fp64 oracle.  Definition:
"AIGC 基本功｜算子融合与 CUDA Graph-Fusion", section 3.5 and the appendix's
attention-tail section.

Bar: |out - ref| <= 1e-2 absolute; the causal zero pattern exact; rows of the
fp32-output mode sum to 1 within 1e-3; bf16 rows within 1e-3 plus half an
ulp per stored entry; tiles visited per row exact.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gemm_epilogues_amd as fc  # noqa: E402
from gpu_util import bf16_from_bits, bits, announce  # noqa: E402

SCALE = float(np.float32(1.0 / np.sqrt(128.0)))


def bf16_vals(u16):
    return synth.bf16_bits_to_f32(u16).astype(np.float64)


def bf16_half_ulp(v):
    """Half an ulp of bf16 at each (non-negative) value."""
    v = np.maximum(np.abs(v), 2.0 ** -126)
    e = np.floor(np.log2(v))
    return 0.5 * 2.0 ** (e - 7)


def check_against_ref(out_bits, ref, S):
    out = bf16_vals(out_bits)
    assert np.max(np.abs(out - ref)) <= 1e-2
    iu = np.triu_indices(S, 1)
    il = np.tril_indices(S)
    o3 = out.reshape(-1, S, S)
    assert np.all(o3[:, iu[0], iu[1]] == 0.0)
    assert np.all(o3[:, il[0], il[1]] > 0.0)
    sums = o3.sum(axis=2)
    slack = 1e-3 + bf16_half_ulp(o3).sum(axis=2)
    assert np.all(np.abs(sums - 1.0) <= slack)


def run_fused(s_dev, BH, S, tile, f32=False):
    if f32:
        out = torch.empty((BH, S, S), dtype=torch.float32, device="cuda")
        fc.fc_causal_softmax_f32out(s_dev, out, SCALE, tile)
        torch.cuda.synchronize()
        return out.cpu().numpy()
    out = torch.empty((BH, S, S), dtype=torch.bfloat16, device="cuda")
    fc.fc_causal_softmax(s_dev, out, SCALE, tile, fc.FC_SOFTMAX_FUSED)
    torch.cuda.synchronize()
    return bits(out)


def run_unfused(s_dev, BH, S):
    out = torch.empty((BH, S, S), dtype=torch.bfloat16, device="cuda")
    wsb = fc.fc_softmax_workspace_bytes(BH, S, fc.FC_SOFTMAX_UNFUSED)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    fc.fc_causal_mask_materialise(ws, BH, S)
    fc.fc_causal_softmax(s_dev, out, SCALE, 64, fc.FC_SOFTMAX_UNFUSED, ws)
    torch.cuda.synchronize()
    mask = ws[: 2 * BH * S * S].view(torch.int16).cpu().numpy().view(np.uint16).reshape(BH, S, S)
    return bits(out), mask


SHAPES = [(1, 1), (2, 2), (1, 3), (2, 63), (1, 64), (2, 65), (1, 129), (3, 256), (1, 640), (2, 1000),
          (1, 1024), (2, 2048)]


@pytest.mark.parametrize("BH,S", SHAPES)
def test_fused_every_tile(BH, S):
    announce(f"softmax fused BH={BH} S={S}")
    s = synth.softmax_inputs(BH, S, salt=S)
    ref = oracle.causal_softmax_f64(s, SCALE)
    sd = bf16_from_bits(s)
    for tile in (64, 128, 256, S):
        check_against_ref(run_fused(sd, BH, S, tile), ref, S)


@pytest.mark.parametrize("BH,S", [(1, 1), (2, 65), (1, 640), (2, 2048)])
def test_fused_f32_rows_sum_to_one(BH, S):
    announce(f"softmax fused f32out BH={BH} S={S}")
    s = synth.softmax_inputs(BH, S, salt=S + 1)
    ref = oracle.causal_softmax_f64(s, SCALE)
    out = run_fused(bf16_from_bits(s), BH, S, 64, f32=True).astype(np.float64)
    assert np.max(np.abs(out - ref)) <= 1e-4
    assert np.all(np.abs(out.sum(axis=2) - 1.0) <= 1e-3)


@pytest.mark.parametrize("BH,S", [(1, 3), (2, 65), (1, 640), (1, 2048)])
def test_tiles_visited_exact(BH, S):
    announce(f"softmax tiles BH={BH} S={S}")
    s = synth.softmax_inputs(BH, S, salt=3)
    sd = bf16_from_bits(s)
    for tile in (64, 128, 256, S):
        out = torch.empty((BH, S, S), dtype=torch.bfloat16, device="cuda")
        cnt = torch.full((BH * S,), -1, dtype=torch.int32, device="cuda")
        fc.fc_causal_softmax_tiles(sd, out, cnt, SCALE, tile)
        torch.cuda.synchronize()
        i = np.tile(np.arange(S), BH)
        assert np.array_equal(cnt.cpu().numpy(), i // tile + 1)
        assert np.array_equal(bits(out), run_fused(sd, BH, S, tile))


@pytest.mark.parametrize("BH,S", [(1, 1), (2, 3), (2, 65), (1, 129), (1, 640), (2, 1000), (2, 2048)])
def test_unfused_baseline(BH, S):
    announce(f"softmax unfused BH={BH} S={S}")
    s = synth.softmax_inputs(BH, S, salt=S + 2)
    ref = oracle.causal_softmax_f64(s, SCALE)
    out, mask = run_unfused(bf16_from_bits(s), BH, S)
    m01 = oracle.causal_mask01(S)
    assert np.array_equal(bf16_vals(mask), np.broadcast_to(m01, (BH, S, S)))
    o = bf16_vals(out)
    assert np.max(np.abs(o - ref)) <= 1e-2
    assert np.all(o.reshape(-1, S, S)[:, m01 == 0] == 0.0)


@pytest.mark.parametrize("fill", [3000.0, np.inf, np.nan])
def test_masked_scores_never_reach_the_result(fill):
    """Scores above the diagonal far above the kept ones (3000, a scaled logit
    about 265 above them), +inf or NaN: the fused kernel (every tile) and the
    unfused baseline still give the oracle's result, which never reads them."""
    announce(f"softmax masked scores = {fill}")
    BH, S = 2, 200
    s = synth.softmax_inputs(BH, S, salt=17)
    iu = np.triu_indices(S, 1)
    s[:, iu[0], iu[1]] = synth.f32_to_bf16_bits(np.array([fill], np.float32))[0]
    ref = oracle.causal_softmax_f64(s, SCALE)
    assert np.isfinite(ref).all()
    sd = bf16_from_bits(s)
    outs = [run_fused(sd, BH, S, tile) for tile in (64, 128, 256, S)]
    outs.append(run_unfused(sd, BH, S)[0])
    for o in outs:
        v = bf16_vals(o)
        assert np.isfinite(v).all()
        assert np.max(np.abs(v - ref)) <= 1e-2
        assert np.all(v.reshape(BH, S, S)[:, iu[0], iu[1]] == 0.0)


def test_special_rows():
    """Row 0 is exactly [1, 0, ...]; equal scores give 1/(i+1) (bf16-rounded)."""
    announce("softmax special rows")
    S = 129
    s = np.full((1, S, S), synth.f32_to_bf16_bits(np.float32(3.0)), dtype=np.uint16)
    out = bf16_vals(run_fused(bf16_from_bits(s), 1, S, 64)).reshape(S, S)
    assert out[0, 0] == 1.0 and np.all(out[0, 1:] == 0.0)
    for i in range(S):
        expect = bf16_vals(synth.f32_to_bf16_bits(np.float32(1.0 / (i + 1))))
        assert np.all(np.abs(out[i, : i + 1] - expect) <= bf16_half_ulp(expect) * 2 + 1e-7)


def check_chunk(o, ref, kept, bf16):
    """One block of rows on the device, in fp64: |out - ref| <= 1e-2 (bf16) or
    1e-4 (fp32 output); exact zeros above the diagonal and positive entries on
    and below it; row sums within 1e-3, plus half a bf16 ulp of every stored
    entry for bf16 output (each stored value is the exact one rounded once)."""
    err = float((o - ref).abs().max())
    assert err <= (1e-2 if bf16 else 1e-4), err
    assert not bool((o[~kept] != 0).any())
    assert bool((o[kept] > 0).all())
    dev1 = (o.sum(1) - 1.0).abs()
    if bf16:
        _, e = torch.frexp(o)                      # o = m 2^e, m in [0.5, 1): ulp = 2^(e-8)
        half = torch.where(o > 0, torch.exp2((e - 9).double()), torch.zeros_like(o))
        slack = 1e-3 + half.sum(1)
    else:
        slack = torch.full_like(dev1, 1e-3)
    worst = float((dev1 - slack).max())
    assert worst <= 0.0, worst


def check_all_rows(s, BH, S, bf16_outs=(), f32_outs=(), chunk_elems=1 << 24):
    """Every row of every output against the fp64 oracle, in blocks of rows
    (the oracle computes a block on the host threads; the comparison runs on
    the device)."""
    total = BH * S
    rows_per = max(1, chunk_elems // S)
    j = torch.arange(S, device="cuda")
    for r0 in range(0, total, rows_per):
        r1 = min(total, r0 + rows_per)
        rid = np.arange(r0, r1, dtype=np.int64)
        ref = torch.from_numpy(oracle.causal_softmax_rows(s, SCALE, rid)).cuda()
        kept = j[None, :] <= torch.from_numpy(rid % S).cuda()[:, None]
        for o in bf16_outs:
            check_chunk(o.view(total, S)[r0:r1].double(), ref, kept, True)
        for o in f32_outs:
            check_chunk(o.view(total, S)[r0:r1].double(), ref, kept, False)
        del ref, kept


@pytest.fixture(scope="module")
def full_scores():
    BH, S = 128, 2048
    announce("softmax full config: generating [8,16,2048,2048] bf16")
    s = synth.softmax_inputs(BH, S)
    return s, bf16_from_bits(s)


def test_full_config_every_row(full_scores):
    """[8,16,2048,2048] bf16, every row of the fused kernel at tiles 64 / 128 /
    256 / none, of its fp32-output mode (tile 64) and of the unfused five-step
    baseline against the fp64 oracle: elementwise within 1e-2 (1e-4 for fp32
    output), the zero pattern exact, and every row's sum within 1e-3 (plus half
    a bf16 ulp per stored entry for bf16 output)."""
    s, sd = full_scores
    BH, S = 128, 2048
    outs = []
    for tile in (64, 128, 256, 2048):
        announce(f"softmax full config fused tile={tile}")
        out = torch.empty((BH, S, S), dtype=torch.bfloat16, device="cuda")
        fc.fc_causal_softmax(sd, out, SCALE, tile, fc.FC_SOFTMAX_FUSED)
        outs.append(out)
    announce("softmax full config unfused")
    out = torch.empty((BH, S, S), dtype=torch.bfloat16, device="cuda")
    wsb = fc.fc_softmax_workspace_bytes(BH, S, fc.FC_SOFTMAX_UNFUSED)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    fc.fc_causal_mask_materialise(ws, BH, S)
    fc.fc_causal_softmax(sd, out, SCALE, 64, fc.FC_SOFTMAX_UNFUSED, ws)
    outs.append(out)
    announce("softmax full config fused fp32 output")
    o32 = torch.empty((BH, S, S), dtype=torch.float32, device="cuda")
    fc.fc_causal_softmax_f32out(sd, o32, SCALE, 64)
    torch.cuda.synchronize()
    del ws
    announce("softmax full config: comparing every row with the oracle")
    check_all_rows(s, BH, S, bf16_outs=outs, f32_outs=[o32])


@pytest.mark.parametrize("S,tile", [(8192, 64), (8192, 8192), (8200, 256), (12288, 128)])
def test_long_rows_every_row(S, tile):
    """The register-resident kernel's longest rows (S = 8192) and the generic
    kernel past it (S > 8192): every row against the oracle with the same bars."""
    announce(f"softmax long rows S={S} tile={tile}")
    s = synth.softmax_inputs(1, S, salt=S + tile)
    sd = bf16_from_bits(s)
    out = torch.empty((1, S, S), dtype=torch.bfloat16, device="cuda")
    fc.fc_causal_softmax(sd, out, SCALE, tile, fc.FC_SOFTMAX_FUSED)
    torch.cuda.synchronize()
    check_all_rows(s, 1, S, bf16_outs=[out])


def random_softmax_shapes():
    rng = np.random.default_rng(20261002 + 1)
    return [(int(rng.integers(1, 4)), int(rng.integers(1, 1400))) for _ in range(8)]


@pytest.mark.parametrize("BH,S", random_softmax_shapes())
def test_random_shapes_every_row(BH, S):
    """Seeded random head counts and row lengths (most not a multiple of any
    tile or of 8, so the generic kernel runs beside the vector one): the fused
    form at every tile and the unfused baseline, every row against the oracle."""
    announce(f"softmax random shape BH={BH} S={S}")
    s = synth.softmax_inputs(BH, S, salt=BH * 7919 + S)
    ref = oracle.causal_softmax_f64(s, SCALE)
    sd = bf16_from_bits(s)
    for tile in (64, 128, 256, S):
        check_against_ref(run_fused(sd, BH, S, tile), ref, S)
    out, _ = run_unfused(sd, BH, S)
    check_against_ref(out, ref, S)
