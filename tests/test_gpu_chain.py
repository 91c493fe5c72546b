"""GPU parity of the K-stage pointwise chain (naive / fused / fat) against the
oracle.  Stage operation: "C-05. Kernel Fusion 代价边界", section 3.

Bar: normwise relative error <= 1e-6 against the fp64 oracle; additionally the
values equal the oracle's one-rounding-per-stage fp32 chain exactly and the
three modes are bit-identical to each other.
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
from gpu_util import f32, host_f32, normwise, announce  # noqa: E402


def run(x_dev, a, b, relu, mode, fat_temps=0, inplace=False):
    n = x_dev.numel()
    y = x_dev.clone() if inplace else torch.empty_like(x_dev)
    src = y if inplace else x_dev
    need = fc.fc_chain_scratch_floats(n, len(a), mode, fat_temps)
    scratch = torch.empty(max(need, 1), dtype=torch.float32, device=x_dev.device) if need else None
    fc.fc_chain(src, y, a, b, relu, mode, scratch, fat_temps)
    torch.cuda.synchronize()
    return host_f32(y), (host_f32(scratch) if scratch is not None else None)


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 1025, 4099, 65536 + 7])
@pytest.mark.parametrize("K", [1, 2, 3, 4, 6, 8])
@pytest.mark.parametrize("relu", [True, False])
def test_chain_modes_small(n, K, relu):
    announce(f"chain n={n} K={K} relu={relu}")
    x, a, b = synth.chain_inputs(n, K, salt=n + K)
    ref64 = oracle.chain_f64(x, a, b, relu)
    ref32 = oracle.chain_f32fma(x, a, b, relu)
    xd = f32(x)
    ys = {}
    for mode in (fc.FC_CHAIN_NAIVE, fc.FC_CHAIN_FUSED, fc.FC_CHAIN_FAT):
        y, _ = run(xd, a, b, relu, mode, fat_temps=16 if mode == fc.FC_CHAIN_FAT else 0)
        ys[mode] = y
        assert np.array_equal(y, ref32), (mode, np.flatnonzero(y != ref32)[:5])
        if np.max(np.abs(ref64)) > 0:
            assert normwise(y, ref64) <= 1e-6
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
    assert np.array_equal(ys[1].view(np.uint32), ys[2].view(np.uint32))


def test_chain_k32_and_odd_stage_counts():
    for K in (5, 7, 13, 32):
        announce(f"chain K={K}")
        x, a, b = synth.chain_inputs(10007, K, salt=K)
        xd = f32(x)
        for mode in (fc.FC_CHAIN_NAIVE, fc.FC_CHAIN_FUSED):
            y, _ = run(xd, a, b, True, mode)
            assert np.array_equal(y, oracle.chain_f32fma(x, a, b, True))


def test_chain_in_place():
    announce("chain in place")
    x, a, b = synth.chain_inputs(4097, 3, salt=9)
    xd = f32(x)
    for mode in (fc.FC_CHAIN_NAIVE, fc.FC_CHAIN_FUSED):
        y, _ = run(xd, a, b, True, mode, inplace=True)
        assert np.array_equal(y, oracle.chain_f32fma(x, a, b, True))


def test_chain_empty_is_noop():
    a = np.ones(2, np.float32)
    fc.fc_chain(torch.empty(0, device="cuda"), torch.empty(0, device="cuda"), a, a)
    torch.cuda.synchronize()


def test_affine_chain_config():
    """8-stage h <- 1.01 h + 0.01 on 1,048,576 fp32 elements, fused vs 8
    single-stage kernels, checked against the collapsed closed form."""
    announce("affine chain n=1048576")
    n = 1048576
    x, a, b = synth.affine_inputs(n)
    A, B = float(a[0]), float(b[0])
    from fractions import Fraction
    Af, Bf = Fraction(A), Fraction(B)
    Ak = float(Af ** 8)
    Bk = float(Bf * (Af ** 8 - 1) / (Af - 1))
    closed = x.astype(np.float64) * Ak + Bk
    xd = f32(x)
    for mode in (fc.FC_CHAIN_FUSED, fc.FC_CHAIN_NAIVE):
        y, _ = run(xd, a, b, False, mode)
        err = normwise(y, closed)
        assert err <= 1e-6, err
        assert normwise(y, oracle.chain_f64(x, a, b, False)) <= 1e-6


@pytest.mark.parametrize("K", [2, 3, 4, 6, 8])
def test_relu_chain_config_full_size(K):
    """n = 16,777,216 fp32, K in {2,3,4,6,8}: naive and fused equal the oracle."""
    announce(f"relu chain n=16777216 K={K}")
    n = 16777216
    x, a, b = synth.chain_inputs(n, K)
    ref32 = oracle.chain_f32fma(x, a, b, True)
    ref64 = oracle.chain_f64(x, a, b, True)
    xd = f32(x)
    for mode in (fc.FC_CHAIN_FUSED, fc.FC_CHAIN_NAIVE):
        y, _ = run(xd, a, b, True, mode)
        assert np.array_equal(y, ref32)
        assert normwise(y, ref64) <= 1e-6
        if K % 2 == 1:
            assert (y >= 0).all()          # last stage is even -> ReLU


def lanes_of(n, K, temps):
    """Lanes of the fat launch: the sink holds one fp32x4 per lane."""
    return fc.fc_chain_scratch_floats(n, K, fc.FC_CHAIN_FAT, temps) // 4


def check_fat(x, a, b, relu, temps, xd=None):
    """Fat y equals the oracle's one-rounding chain bit for bit (and the fp64
    chain normwise within 1e-6); the sink equals the oracle's fp32 evaluation
    of its formula exactly and the fp64 one within 64 u of the sum of
    |t_j| (T + K + the lane's vector count roundings, each at most u of it)."""
    n, K = x.size, a.size
    xd = f32(x) if xd is None else xd
    y, sink = run(xd, a, b, relu, fc.FC_CHAIN_FAT, fat_temps=temps)
    ref32 = oracle.chain_f32fma(x, a, b, relu)
    assert np.array_equal(y, ref32), np.flatnonzero(y != ref32)[:5]
    assert normwise(y, oracle.chain_f64(x, a, b, relu)) <= 1e-6
    lanes = lanes_of(n, K, temps)
    assert sink.size == 4 * lanes
    s32 = oracle.chain_fat_sink_f32(x, a, b, relu, temps, lanes)
    # values, not bits: a ReLU may leave -0.0 or +0.0 (either is accepted)
    bad = np.flatnonzero(~(sink == s32))
    assert bad.size == 0, (bad[:5], sink[bad[:5]], s32[bad[:5]])
    s64, absd = oracle.chain_fat_sink_f64(x, a, b, relu, temps, lanes, with_abs=True)
    assert np.all(np.abs(sink.astype(np.float64) - s64) <= 64 * 2.0 ** -24 * absd + 1e-30)
    if temps:
        assert np.abs(sink).sum() > 0


@pytest.mark.parametrize("temps", [0, 16, 48, 96, 128])
def test_fat_probe_small_with_tail(temps):
    """K = 4 fat probe on 2^20 + 5 elements (a ragged tail the sink skips):
    y and the sink against the oracle, y bit-identical to the fused kernel."""
    announce(f"fat K=4 temps={temps} n=2^20+5")
    n = (1 << 20) + 5
    x, a, b = synth.chain_inputs(n, 4, salt=77)
    xd = f32(x)
    check_fat(x, a, b, True, temps, xd)
    yf, _ = run(xd, a, b, True, fc.FC_CHAIN_FUSED)
    yt, _ = run(xd, a, b, True, fc.FC_CHAIN_FAT, fat_temps=temps)
    assert np.array_equal(yf.view(np.uint32), yt.view(np.uint32))


@pytest.fixture(scope="module")
def full_chain_inputs():
    cache = {}

    def get(K):
        if K not in cache:
            announce(f"generating chain inputs n=16777216 K={K}")
            x, a, b = synth.chain_inputs(16777216, K)
            cache.clear()
            cache[K] = (x, a, b, f32(x))
        return cache[K]
    return get


@pytest.mark.parametrize("K,temps", [(4, 0), (4, 16), (4, 48), (4, 96), (4, 128),
                                     (2, 48), (3, 48), (6, 48), (8, 48)])
def test_fat_probe_full_size(full_chain_inputs, K, temps):
    """n = 16,777,216 (the chain workload): the fat probe at the T sweep's
    points (K = 4) and at T = 48 for every K, y and sink against the oracle."""
    announce(f"fat full size n=16777216 K={K} temps={temps}")
    x, a, b, xd = full_chain_inputs(K)
    check_fat(x, a, b, True, temps, xd)


def random_chain_cases():
    rng = np.random.default_rng(20261002 + 4)
    return [(int(rng.integers(1, 400000)), int(rng.integers(1, 33)), bool(rng.integers(0, 2))) for _ in range(10)]


@pytest.mark.parametrize("n,K,relu", random_chain_cases())
def test_random_lengths_and_stage_counts(n, K, relu):
    """Seeded random lengths (ragged tails) and stage counts 1..32: naive and
    fused equal the oracle's one-rounding chain bit for bit, and the fat probe
    (where it supports K) its y and sink."""
    announce(f"chain random n={n} K={K} relu={relu}")
    x, a, b = synth.chain_inputs(n, K, salt=n + K)
    ref32 = oracle.chain_f32fma(x, a, b, relu)
    xd = f32(x)
    for mode in (fc.FC_CHAIN_NAIVE, fc.FC_CHAIN_FUSED):
        y, _ = run(xd, a, b, relu, mode)
        assert np.array_equal(y, ref32), mode
    if K in (1, 2, 3, 4, 6, 8):
        check_fat(x, a, b, relu, 48, xd)
