"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, its integer accounting equals the oracle's stage-walking
ledgers (and the values the pages print), and invalid arguments are rejected
before any HIP call.

Every validation case below is invalid by construction, so no kernel is ever
launched from this file (the pointers are fake host addresses).
"""
import ctypes
import os
import re

import pytest

import gemm_epilogues_amd as fc
from oracle import ledger
from conftest import load_golden

FAKE = 0x10000          # a 16-byte aligned address that is never dereferenced
MIS = 0x10004           # misaligned


def declared_symbols():
    text = open(fc.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fc_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 15
    lib = ctypes.CDLL(fc.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fc.EXPORTED)
    assert "gfx950" in fc.fc_version()


def test_status_strings():
    for code in range(0, -9, -1):
        assert fc.fc_status_string(code) != "unknown status"
    assert fc.fc_status_string(-99) == "unknown status"


def test_plan_accounting_matches_ledger_and_page():
    g = load_golden("k4_split_plans.json")
    for row in g["plans"]:
        assert fc.fc_plan_bytes(4096, 4096, 4096, row["plan"]) == row["bytes"]
        assert fc.fc_plan_launches(row["plan"]) == row["launches"]
    for M, N, K in [(16, 4096, 4096), (1, 8, 8), (17, 40, 24), (4096, 4096, 4096), (300, 1000, 72),
                    (1, 2048, 2048), (16, 64, 65536), (8, 640, 768), (3, 128, 256)]:
        for plan in ledger.compositions(4):
            assert fc.fc_plan_bytes(M, N, K, plan) == ledger.plan_bytes(M, N, K, plan)
            assert fc.fc_plan_bytes(M, N, K, plan, 4) == ledger.plan_bytes(M, N, K, plan, 4)
            assert fc.fc_plan_launches(plan) == ledger.plan_launches(plan) == len(plan)
            ws = fc.fc_gemm_workspace_bytes(M, N, K, plan)
            assert ws == (-(-2 * M * N // 256) * 256 if len(plan) > 1 else 0) + decode_scratch(M, N, K)


def decode_scratch(M, N, K):
    """Workspace the split-K decode kernel adds, per the header: for M <= 16,
    N % 64 == 0, K % 256 == 0, P is the smallest power of two with at most 4
    32-deep k-steps per wave (K <= 1024 P) that gives N/64 * P >= 512
    workgroups (else the largest such P, up to 64, with 256 P dividing K)."""
    if M > 16 or N % 64 or K % 256:
        return 0
    strips, best, P = N // 64, 0, 1
    while P <= 64 and K % (256 * P) == 0:
        if K <= 1024 * P:
            best = P
            if strips * P >= 512:
                break
        P *= 2
    if best <= 1:
        return 0
    return -(-4 * strips // 256) * 256 + strips * best * 16 * 64 * 4


def test_decode_workspace_examples():
    # 16x4096x4096: 64 strips x 8 splits = 512 workgroups
    assert fc.fc_gemm_workspace_bytes(16, 4096, 4096, [4]) == 256 + 64 * 8 * 4096
    assert fc.fc_gemm_workspace_bytes(16, 4096, 4096, [1, 3]) == 256 + 64 * 8 * 4096 + 131072
    # 1x2048x2048: 32 strips x 8 splits (256 P must divide K)
    assert fc.fc_gemm_workspace_bytes(1, 2048, 2048, [4]) == 256 + 32 * 8 * 4096
    # N = 16384, K = 1024: 256 strips x 2 splits
    assert fc.fc_gemm_workspace_bytes(16, 16384, 1024, [4]) == 1024 + 256 * 2 * 4096
    # N = 32768: 512 strips fill the chip unsplit, no scratch
    assert fc.fc_gemm_workspace_bytes(16, 32768, 1024, [4]) == 0
    # 17..32 rows: two 16-row blocks of partials; 33..64 rows: four (and at
    # most 2 k-steps per wave, so 4096 deep needs P >= 8)
    assert fc.fc_gemm_workspace_bytes(17, 4096, 4096, [4]) == 256 + 64 * 8 * 2 * 4096
    assert fc.fc_gemm_workspace_bytes(32, 4096, 4096, [4]) == 256 + 64 * 8 * 2 * 4096
    assert fc.fc_gemm_workspace_bytes(64, 4096, 4096, [4]) == 256 + 64 * 8 * 4 * 4096
    assert fc.fc_gemm_workspace_bytes(40, 2048, 8192, [4]) == 256 + 32 * 16 * 4 * 4096
    # shapes the decode kernel does not take: from 65 rows the 128x128 ring
    # kernel (32 tiles, K split 4 ways)
    assert fc.fc_gemm_workspace_bytes(65, 4096, 4096, [4]) == 256 + 32 * 4 * 128 * 128 * 4
    assert fc.fc_gemm_workspace_bytes(16, 4104, 4096, [4]) == 0
    assert fc.fc_gemm_workspace_bytes(16, 4096, 4104, [4]) == 0


def test_ring128_split_workspace_examples():
    tile = 128 * 128 * 4                       # one fp32 partial tile
    # 129 rows: 2 x 32 tiles of 128x128, K split 2 ways -> 128 workgroups
    assert fc.fc_gemm_workspace_bytes(129, 4096, 4096, [4]) == 256 + 64 * 2 * tile
    assert fc.fc_gemm_workspace_bytes(129, 4096, 4096, [2, 2]) == 256 + 64 * 2 * tile + 2 * 129 * 4096
    # 200 x 2048: 32 tiles, 4 ways; 1024^3: 64 tiles, 2 ways
    assert fc.fc_gemm_workspace_bytes(200, 2048, 2048, [4]) == 256 + 32 * 4 * tile
    assert fc.fc_gemm_workspace_bytes(1024, 1024, 1024, [4]) == 256 + 64 * 2 * tile
    # 300 x 1000 x 1024: 24 tiles; a split must stay >= 256 deep, so P = 4
    assert fc.fc_gemm_workspace_bytes(300, 1000, 1024, [4]) == 256 + 24 * 4 * tile
    # 128..512 tiles of 128x128, or more than 512 (the 256x256 ring kernel): no split
    assert fc.fc_gemm_workspace_bytes(512, 4096, 4096, [4]) == 0
    assert fc.fc_gemm_workspace_bytes(2048, 4096, 4096, [4]) == 0
    assert fc.fc_gemm_workspace_bytes(4096, 4096, 4096, [4]) == 0
    # too shallow to split (K / 2 < 256), or K % 64 != 0 (register-staged kernels)
    assert fc.fc_gemm_workspace_bytes(129, 4096, 256, [4]) == 0
    assert fc.fc_gemm_workspace_bytes(129, 4096, 4000, [4]) == 0


@pytest.mark.parametrize("plan", [[], [0, 4], [5], [1, 1, 1], [2, -1, 3], [1, 1, 1, 1, 0]])
def test_bad_plan_accounting_is_zero(plan):
    assert fc.fc_plan_bytes(16, 16, 16, plan) == 0
    assert fc.fc_plan_launches(plan) == 0
    assert fc.fc_gemm_workspace_bytes(16, 16, 16, plan) == 0


def test_chain_accounting_matches_ledger():
    for n in (0, 1, 5, 1048576, 16777216):
        for K in (1, 2, 3, 4, 6, 8, 32):
            assert fc.fc_chain_bytes(n, K, fc.FC_CHAIN_NAIVE) == ledger.chain_bytes(n, K, False)
            assert fc.fc_chain_bytes(n, K, fc.FC_CHAIN_FUSED) == ledger.chain_bytes(n, K, True)
            assert fc.fc_chain_bytes(n, K, fc.FC_CHAIN_FAT) == ledger.chain_bytes(n, K, True)
            assert fc.fc_chain_bytes(n, K, fc.FC_CHAIN_NAIVE) == K * fc.fc_chain_bytes(n, K, fc.FC_CHAIN_FUSED)


def test_softmax_accounting_matches_ledger():
    for BH, S in [(1, 1), (2, 3), (3, 63), (1, 64), (2, 65), (1, 129), (4, 300), (128, 2048)]:
        for tile in (64, 128, 256, S):
            assert fc.fc_softmax_bytes(BH, S, tile, fc.FC_SOFTMAX_FUSED) == \
                ledger.softmax_bytes(BH, S, tile, True), (BH, S, tile)
        assert fc.fc_softmax_bytes(BH, S, 64, fc.FC_SOFTMAX_UNFUSED) == ledger.softmax_bytes(BH, S, 64, False)
    assert fc.fc_softmax_bytes(128, 2048, 64, fc.FC_SOFTMAX_FUSED) == 1627389952
    assert fc.fc_softmax_bytes(128, 2048, 2048, fc.FC_SOFTMAX_FUSED) == 2 * 1024 ** 3
    assert fc.fc_softmax_bytes(128, 2048, 32, fc.FC_SOFTMAX_FUSED) == 0


def test_workspace_sizes():
    assert fc.fc_softmax_workspace_bytes(128, 2048, fc.FC_SOFTMAX_FUSED) == 0
    assert fc.fc_softmax_workspace_bytes(128, 2048, fc.FC_SOFTMAX_UNFUSED) == 2 * 128 * 2048 ** 2 + 8 * 128 * 2048
    assert fc.fc_softmax_workspace_bytes(1, 3, fc.FC_SOFTMAX_UNFUSED) == 256 + 8 * 3
    assert fc.fc_chain_scratch_floats(1000, 4, fc.FC_CHAIN_NAIVE) == 1000
    assert fc.fc_chain_scratch_floats(1000, 1, fc.FC_CHAIN_NAIVE) == 0
    assert fc.fc_chain_scratch_floats(1000, 4, fc.FC_CHAIN_FUSED) == 0
    assert fc.fc_chain_scratch_floats(1 << 24, 4, fc.FC_CHAIN_FAT, 48) == 2048 * 256 * 4


# ---------------------------------------------------------------- validation (no HIP call)

def _f32(vals):
    import numpy as np
    a = np.asarray(vals, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


L = fc.lib()


def test_chain_validation():
    a, ap = _f32([1.0, 2.0])
    b, bp = _f32([0.0, 0.0])
    # negative n
    assert L.fc_chain(FAKE, FAKE, -1, ap, bp, 2, 1, fc.FC_CHAIN_FUSED, None, 0, None) == fc.FC_ERR_SHAPE
    # K out of range
    assert L.fc_chain(FAKE, FAKE, 8, ap, bp, 0, 1, fc.FC_CHAIN_FUSED, None, 0, None) == fc.FC_ERR_UNSUPPORTED
    assert L.fc_chain(FAKE, FAKE, 8, ap, bp, 33, 1, fc.FC_CHAIN_FUSED, None, 0, None) == fc.FC_ERR_UNSUPPORTED
    # bad mode
    assert L.fc_chain(FAKE, FAKE, 8, ap, bp, 2, 1, 7, None, 0, None) == fc.FC_ERR_UNSUPPORTED
    # null coefficients / data
    assert L.fc_chain(FAKE, FAKE, 8, None, bp, 2, 1, fc.FC_CHAIN_FUSED, None, 0, None) == fc.FC_ERR_NULL
    assert L.fc_chain(None, FAKE, 8, ap, bp, 2, 1, fc.FC_CHAIN_FUSED, None, 0, None) == fc.FC_ERR_NULL
    # misaligned
    assert L.fc_chain(MIS, FAKE + 4096, 8, ap, bp, 2, 1, fc.FC_CHAIN_FUSED, None, 0, None) == fc.FC_ERR_ALIGN
    # partial overlap of x and y
    assert L.fc_chain(FAKE, FAKE + 16, 8, ap, bp, 2, 1, fc.FC_CHAIN_FUSED, None, 0, None) == fc.FC_ERR_ALIAS
    # naive without scratch / misaligned scratch / overlapping scratch
    assert L.fc_chain(FAKE, FAKE + 4096, 8, ap, bp, 2, 1, fc.FC_CHAIN_NAIVE, None, 0, None) == fc.FC_ERR_WORKSPACE
    assert L.fc_chain(FAKE, FAKE + 4096, 8, ap, bp, 2, 1, fc.FC_CHAIN_NAIVE, MIS + 8192, 0, None) == fc.FC_ERR_ALIGN
    assert L.fc_chain(FAKE, FAKE + 4096, 8, ap, bp, 2, 1, fc.FC_CHAIN_NAIVE, FAKE + 16, 0, None) == fc.FC_ERR_ALIAS
    # fat: unsupported temps / stages
    assert L.fc_chain(FAKE, FAKE + 4096, 8, ap, bp, 2, 1, fc.FC_CHAIN_FAT, FAKE + 8192, 7, None) == fc.FC_ERR_UNSUPPORTED
    a5, ap5 = _f32([1.0] * 5)
    assert L.fc_chain(FAKE, FAKE + 4096, 8, ap5, ap5, 5, 1, fc.FC_CHAIN_FAT, FAKE + 8192, 48, None) == fc.FC_ERR_UNSUPPORTED
    a2, _ = a, b
    assert L.fc_chain(FAKE, FAKE + 4096, 8, ap, bp, 2, 1, fc.FC_CHAIN_FAT, FAKE + 8192, 96, None) == fc.FC_ERR_UNSUPPORTED
    # n == 0 is a no-op that enqueues nothing
    assert L.fc_chain(None, None, 0, ap, bp, 2, 1, fc.FC_CHAIN_FUSED, None, 0, None) == fc.FC_OK


def _plan(p):
    arr = (ctypes.c_int * max(1, len(p)))(*p)
    return arr, len(p)


def test_gemm_validation():
    p4, n4 = _plan([4])
    p13, n13 = _plan([1, 3])
    A, B, bias, R, Y = FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (3 << 20), FAKE + (4 << 20)
    W = FAKE + (5 << 20)
    for bad in ([0, 4], [5], [1, 1, 1], [], [1, 1, 1, 1, 0]):
        pb, nb = _plan(bad)
        assert L.fc_gemm_epilogue(A, B, bias, R, Y, 16, 64, 64, pb, nb, W, 1 << 20, None) == fc.FC_ERR_PLAN
    assert L.fc_gemm_epilogue(A, B, bias, R, Y, 16, 64, 64, None, 1, W, 1 << 20, None) == fc.FC_ERR_PLAN
    assert L.fc_gemm_epilogue(A, B, bias, R, Y, 0, 64, 64, p4, n4, None, 0, None) == fc.FC_ERR_SHAPE
    assert L.fc_gemm_epilogue(A, B, bias, R, Y, 16, 60, 64, p4, n4, None, 0, None) == fc.FC_ERR_UNSUPPORTED
    assert L.fc_gemm_epilogue(A, B, bias, R, Y, 16, 64, 12, p4, n4, None, 0, None) == fc.FC_ERR_UNSUPPORTED
    assert L.fc_gemm_epilogue(A, B, None, R, Y, 16, 64, 64, p4, n4, None, 0, None) == fc.FC_ERR_NULL
    assert L.fc_gemm_epilogue(A, B, bias, R, MIS, 16, 64, 64, p4, n4, None, 0, None) == fc.FC_ERR_ALIGN
    assert L.fc_gemm_epilogue(A, B, bias, R, R, 16, 64, 64, p4, n4, None, 0, None) == fc.FC_ERR_ALIAS
    assert L.fc_gemm_epilogue(A, B, bias, R, Y, 16, 64, 64, p13, n13, None, 0, None) == fc.FC_ERR_WORKSPACE
    assert L.fc_gemm_epilogue(A, B, bias, R, Y, 16, 64, 64, p13, n13, W, 16 * 64 * 2 - 2, None) == fc.FC_ERR_WORKSPACE
    assert L.fc_gemm_epilogue(A, B, bias, R, Y, 16, 64, 64, p13, n13, MIS + (6 << 20), 1 << 20, None) == fc.FC_ERR_ALIGN
    assert L.fc_gemm_epilogue(A, B, bias, R, Y, 16, 64, 64, p13, n13, Y, 1 << 20, None) == fc.FC_ERR_ALIAS


def test_softmax_validation():
    s, o, w = FAKE, FAKE + (1 << 24), FAKE + (2 << 24)
    assert L.fc_causal_softmax(s, o, 0, 64, 0.1, 64, fc.FC_SOFTMAX_FUSED, None, 0, None) == fc.FC_ERR_SHAPE
    assert L.fc_causal_softmax(s, o, 1, 0, 0.1, 64, fc.FC_SOFTMAX_FUSED, None, 0, None) == fc.FC_ERR_SHAPE
    assert L.fc_causal_softmax(None, o, 1, 64, 0.1, 64, fc.FC_SOFTMAX_FUSED, None, 0, None) == fc.FC_ERR_NULL
    assert L.fc_causal_softmax(MIS, o, 1, 64, 0.1, 64, fc.FC_SOFTMAX_FUSED, None, 0, None) == fc.FC_ERR_ALIGN
    assert L.fc_causal_softmax(s, s + 32, 1, 64, 0.1, 64, fc.FC_SOFTMAX_FUSED, None, 0, None) == fc.FC_ERR_ALIAS
    for tile in (0, 32, 100, 512):
        assert L.fc_causal_softmax(s, o, 1, 1024, 0.1, tile, fc.FC_SOFTMAX_FUSED, None, 0, None) == fc.FC_ERR_UNSUPPORTED
    assert L.fc_causal_softmax(s, o, 1, 64, 0.1, 64, 5, None, 0, None) == fc.FC_ERR_UNSUPPORTED
    need = fc.fc_softmax_workspace_bytes(1, 64, fc.FC_SOFTMAX_UNFUSED)
    assert L.fc_causal_softmax(s, o, 1, 64, 0.1, 64, fc.FC_SOFTMAX_UNFUSED, None, 0, None) == fc.FC_ERR_WORKSPACE
    assert L.fc_causal_softmax(s, o, 1, 64, 0.1, 64, fc.FC_SOFTMAX_UNFUSED, w, need - 1, None) == fc.FC_ERR_WORKSPACE
    assert L.fc_causal_softmax(s, o, 1, 64, 0.1, 64, fc.FC_SOFTMAX_UNFUSED, o, need, None) == fc.FC_ERR_ALIAS
    assert L.fc_causal_softmax_f32out(s, o, 1, 64, 0.1, 48, None) == fc.FC_ERR_UNSUPPORTED
    assert L.fc_causal_softmax_tiles(s, o, None, 1, 64, 0.1, 64, None) == fc.FC_ERR_NULL
    assert L.fc_causal_mask_materialise(None, 1, 4, None) == fc.FC_ERR_NULL
    assert L.fc_causal_mask_materialise(MIS, 1, 4, None) == fc.FC_ERR_ALIGN
    assert L.fc_causal_mask_materialise(FAKE, 0, 4, None) == fc.FC_ERR_SHAPE


# ---------------------------------------------------------------- measurement probes (libfcenv.so)

def test_envelope_library_exports_its_header():
    from gemm_epilogues_amd import envelope as env
    text = open(os.path.join(os.path.dirname(fc.HEADER), "fc_envelope.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(fce_[a-z0-9_]+)\s*\(", text)))
    lib = ctypes.CDLL(env.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(env.EXPORTED)
    assert env.fce_chunk_bytes() == 32768
    assert env.fce_mfma_sink_floats() == 1024 * 256
    assert env.fce_mfma_flops(10) == 1024 * 4 * 10 * 8 * 2 * 32 * 32 * 16
    assert env.fce_mfma_flops(0) == 0.0


def test_envelope_validation_before_launch():
    from gemm_epilogues_amd import envelope as env
    L = env._lib
    C = 32768
    assert L.fce_mix(FAKE, C, None, C, None) == fc.FC_ERR_NULL
    assert L.fce_mix(None, C, FAKE, C, None) == fc.FC_ERR_NULL
    assert L.fce_mix(FAKE, 0, FAKE, 0, None) == fc.FC_ERR_SHAPE
    assert L.fce_mix(FAKE, C, FAKE + 4 * C, C + 16, None) == fc.FC_ERR_SHAPE
    assert L.fce_mix(FAKE, 2 * C, FAKE + 4 * C, C, None) == fc.FC_ERR_SHAPE
    assert L.fce_mix(MIS, C, FAKE + 4 * C, C, None) == fc.FC_ERR_ALIGN
    assert L.fce_mix(FAKE, C, FAKE + C // 2, C, None) == fc.FC_ERR_ALIAS
    assert L.fce_read(None, C, FAKE, None) == fc.FC_ERR_NULL
    assert L.fce_read(FAKE, C + 1, FAKE, None) == fc.FC_ERR_SHAPE
    assert L.fce_read(MIS, C, FAKE, None) == fc.FC_ERR_ALIGN
    assert L.fce_mfma(None, 1, None) == fc.FC_ERR_NULL
    assert L.fce_mfma(FAKE, 0, None) == fc.FC_ERR_SHAPE
    assert L.fce_empty(0, FAKE, None) == fc.FC_ERR_SHAPE
    assert L.fce_empty(4, None, None) == fc.FC_ERR_NULL
    assert L.fce_empty_n(4, 0, FAKE, None) == fc.FC_ERR_SHAPE
    assert L.fce_empty_n(4, 3, None, None) == fc.FC_ERR_NULL
    assert L.fce_mix_n(FAKE, C, FAKE + 4 * C, C, 0, None) == fc.FC_ERR_SHAPE
    assert L.fce_mix_n(FAKE, C, FAKE + C // 2, C, 2, None) == fc.FC_ERR_ALIAS


def test_attention_accounting_and_validation():
    assert fc.fc_attention_flops(1, 1, 128) == 2 * 128 * 1 * 2
    assert fc.fc_attention_flops(128, 2048, 128) == 2 * 128 * 2048 * 2049 * 128
    assert fc.fc_attention_bytes(128, 2048, 128) == 8 * 128 * 2048 * 128
    assert fc.fc_attention_flops(0, 5, 128) == 0 and fc.fc_attention_bytes(1, 0, 128) == 0
    L = fc.lib()
    big = 1 << 24
    assert L.fc_causal_attention(FAKE, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 1, 8, 64, 0.1, None) == fc.FC_ERR_UNSUPPORTED
    far = 1 << 31                                 # S past 2^22: byte offsets inside a head would pass 2^31
    assert L.fc_causal_attention(FAKE, FAKE + far, FAKE + 2 * far, FAKE + 3 * far, 1, (1 << 22) + 1, 128, 0.1,
                                 None) == fc.FC_ERR_UNSUPPORTED
    assert L.fc_causal_attention(FAKE, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 1, 0, 128, 0.1, None) == fc.FC_ERR_SHAPE
    assert L.fc_causal_attention(FAKE, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 0, 8, 128, 0.1, None) == fc.FC_ERR_SHAPE
    for bad in (float("nan"), 0.0, -0.1, float("inf")):
        assert L.fc_causal_attention(FAKE, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 1, 8, 128, bad, None) == fc.FC_ERR_SHAPE
    assert L.fc_causal_attention(None, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 1, 8, 128, 0.1, None) == fc.FC_ERR_NULL
    assert L.fc_causal_attention(MIS, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 1, 8, 128, 0.1, None) == fc.FC_ERR_ALIGN
    assert L.fc_causal_attention(FAKE, FAKE + big, FAKE + 2 * big, FAKE + 1024, 1, 8, 128, 0.1, None) == fc.FC_ERR_ALIAS


def test_rmsnorm_accounting_and_validation():
    n = 1024 * 4096
    assert fc.fc_rmsnorm_bytes(1024, 4096, fc.FC_RMSNORM_FUSED) == 8 * n
    assert fc.fc_rmsnorm_bytes(1024, 4096, fc.FC_RMSNORM_UNFUSED) == 32 * n
    assert fc.fc_rmsnorm_bytes(0, 4096, 0) == 0 and fc.fc_rmsnorm_bytes(4, 4, 7) == 0
    assert fc.fc_rmsnorm_workspace_bytes(1024, 4096, fc.FC_RMSNORM_FUSED) == 0
    assert fc.fc_rmsnorm_workspace_bytes(3, 12, fc.FC_RMSNORM_UNFUSED) == 256 + 12
    L = fc.lib()
    big = 1 << 24
    args = (FAKE, FAKE + big, FAKE + 2 * big)
    assert L.fc_rmsnorm(*args, 4, 6, 1e-5, 0, None, 0, None) == fc.FC_ERR_UNSUPPORTED      # d % 4
    assert L.fc_rmsnorm(*args, 4, 16388, 1e-5, 0, None, 0, None) == fc.FC_ERR_UNSUPPORTED  # d too long
    assert L.fc_rmsnorm(*args, 0, 64, 1e-5, 0, None, 0, None) == fc.FC_ERR_SHAPE
    assert L.fc_rmsnorm(*args, 4, 64, -1.0, 0, None, 0, None) == fc.FC_ERR_SHAPE
    assert L.fc_rmsnorm(*args, 4, 64, float("nan"), 0, None, 0, None) == fc.FC_ERR_SHAPE
    assert L.fc_rmsnorm(*args, 4, 64, 1e-5, 2, None, 0, None) == fc.FC_ERR_UNSUPPORTED
    assert L.fc_rmsnorm(None, FAKE + big, FAKE + 2 * big, 4, 64, 1e-5, 0, None, 0, None) == fc.FC_ERR_NULL
    assert L.fc_rmsnorm(MIS, FAKE + big, FAKE + 2 * big, 4, 64, 1e-5, 0, None, 0, None) == fc.FC_ERR_ALIGN
    assert L.fc_rmsnorm(FAKE, FAKE + big, FAKE + 512, 4, 64, 1e-5, 0, None, 0, None) == fc.FC_ERR_ALIAS
    assert L.fc_rmsnorm(*args, 4, 64, 1e-5, 1, None, 0, None) == fc.FC_ERR_WORKSPACE


def _report_by_plain_name():
    """kernel_resources.json (the compiler's report, keyed by mangled name) keyed
    by demangled name without the parameter list, for the library's kernels."""
    import subprocess
    path = os.path.join(os.path.dirname(fc.__file__), "kernel_resources.json")
    with open(path) as f:
        rep = __import__("json").load(f)
    mangled = sorted(rep)
    plain = subprocess.run(["c++filt"], input="\n".join(mangled), capture_output=True, text=True,
                           check=True).stdout.splitlines()
    out = {}
    for m, full in zip(mangled, plain):
        full = full[5:] if full.startswith("void ") else full
        depth, cut = 0, len(full)
        for i, ch in enumerate(full):
            depth += (ch == "<") - (ch == ">")
            if ch == "(" and depth == 0:
                cut = i
                break
        out[full[:cut]] = rep[m]
    return out


def test_kernel_info_matches_the_compiler_report():
    names = fc.fc_kernel_names()
    assert len(names) == len(set(names)) and names == sorted(names)
    rep = _report_by_plain_name()
    fields = {"vgprs": "VGPRs", "agprs": "AGPRs", "sgprs": "TotalSGPRs", "lds_bytes": "LDS Size [bytes/block]",
              "scratch_bytes": "ScratchSize [bytes/lane]", "waves_per_simd": "Occupancy [waves/SIMD]"}
    for n in names:
        info = fc.fc_kernel_info(n)
        assert {k: info[k] for k in fields} == {k: rep[n][v] for k, v in fields.items()}, n
    # every product kernel is listed; the measurement probes (a separate library) are not
    for key in ("fc::attention_fwd_kernel", "fc::gemm_ring_kernel<3>", "fc::gemm_decode_kernel<3, 1>",
                "fc::chain_fused_kernel<4, true>", "fc::chain_fat_kernel<4, true, 48>", "fc::rmsnorm_fused_kernel<4>"):
        assert key in names, key
    assert not any(n.startswith("fc::fce_") or "envelope" in n for n in names)


def test_kernel_info_shows_the_register_cliff():
    # the fused chain keeps few values live and runs at full occupancy; the fat
    # probe's 48 live fp32x4 temporaries push the registers past 192 and the
    # occupancy down to 2 waves per SIMD, without spilling
    fused = fc.fc_kernel_info("fc::chain_fused_kernel<4, true>")
    fat = fc.fc_kernel_info("fc::chain_fat_kernel<4, true, 48>")
    assert fused["waves_per_simd"] == 8 and fused["scratch_bytes"] == 0
    assert fat["vgprs"] + fat["agprs"] >= 192 and fat["waves_per_simd"] <= 2 and fat["scratch_bytes"] == 0
    att = fc.fc_kernel_info("fc::attention_fwd_kernel")
    assert att["lds_bytes"] == 65536 and att["waves_per_simd"] == 2 and att["scratch_bytes"] == 0


def test_kernel_info_errors():
    assert fc.lib().fc_kernel_info(None, None, None, None, None, None, None) == fc.FC_ERR_NULL
    assert fc.lib().fc_kernel_info(b"fc::no_such_kernel", None, None, None, None, None, None) == \
        fc.FC_ERR_UNSUPPORTED
    with pytest.raises(fc.FcError):
        fc.fc_kernel_info("attention_fwd_kernel")             # the namespace is part of the name
    assert fc.lib().fc_kernel_info(b"fc::attention_fwd_kernel", None, None, None, None, None, None) == fc.FC_OK
    assert fc.lib().fc_kernel_name(-1) is None
    assert fc.lib().fc_kernel_name(len(fc.fc_kernel_names())) is None


def test_headers_compile_as_c_and_answer_from_c(tmp_path):
    """A plain C99 program (tests/c_abi_check.c) built by gcc with -pedantic
    -Werror against include/fc.h and include/fc_envelope.h, linked to the two
    libraries: the declarations are C, and the host-only calls and argument
    validation answer from C as they do through the binding."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    here = os.path.dirname(os.path.abspath(__file__))
    libdir = os.path.dirname(fc.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.dirname(fc.HEADER), os.path.join(here, "c_abi_check.c"),
                    "-L", libdir, "-lfc", "-lfcenv", f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    got = dict(line.split(" ", 1) for line in out.strip().splitlines())
    assert got["version"] == fc.fc_version()
    for name, plan in (("plan_bytes_4", [4]), ("plan_bytes_13", [1, 3]), ("plan_bytes_1111", [1, 1, 1, 1])):
        assert int(got[name]) == ledger.plan_bytes(4096, 4096, 4096, plan)
    assert int(got["plan_launches_1111"]) == 4
    assert int(got["chain_bytes_fused"]) == ledger.chain_bytes(16777216, 8, True)
    assert int(got["chain_bytes_naive"]) == ledger.chain_bytes(16777216, 8, False)
    assert int(got["softmax_bytes_t64"]) == fc.fc_softmax_bytes(128, 2048, 64, fc.FC_SOFTMAX_FUSED)
    assert int(got["workspace_13"]) == fc.fc_gemm_workspace_bytes(4096, 4096, 4096, [1, 3])
    assert int(got["gemm_bad_plan"]) == fc.FC_ERR_PLAN
    assert int(got["gemm_null"]) == fc.FC_ERR_NULL
    assert int(got["noalloc_scratch"]) == fc.FC_ERR_SCRATCH
    assert int(got["chain_k0"]) == fc.FC_ERR_UNSUPPORTED
    assert int(got["softmax_bad_tile"]) == fc.FC_ERR_UNSUPPORTED
    assert int(got["stages"]) == 0 and int(got["kernel_info"]) == 0
    assert int(got["kernel_vgprs"]) == fc.fc_kernel_info("fc::attention_fwd_kernel")["vgprs"]
    assert got["status_scratch"] == fc.fc_status_string(fc.FC_ERR_SCRATCH)
    assert int(got["noalloc_limit"]) == fc.FC_GEMM_NOALLOC_SCRATCH_BYTES
    assert int(got["envelope_bad"]) == fc.FC_ERR_NULL
