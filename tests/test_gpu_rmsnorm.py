"""GPU parity of RMSNorm, fused (one pass) and unfused (the appendix ledger's
four passes), against the fp64 oracle.

Bar, per element: |y - ref| <= 4e-6 |ref|.  Both forms compute in fp32: the
sum of squares over a row (at most 16384 terms, summed in a tree of short
runs) carries a relative error of a few 1e-7, the square root and reciprocal
are correctly rounded, and two products add 1.2e-7.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gemm_epilogues_amd as fc  # noqa: E402
from gpu_util import announce  # noqa: E402


def inputs(rows, d, salt):
    rng = np.random.default_rng(1000 + salt)
    x = rng.standard_normal((rows, d)).astype(np.float32) * np.float32(rng.uniform(0.1, 10.0))
    g = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    return x, g


def run(x, g, eps, mode):
    xd, gd = torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda()
    yd = torch.empty_like(xd)
    fc.fc_rmsnorm(xd, gd, yd, eps, mode)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


@pytest.mark.parametrize("rows,d", [(1, 4), (3, 64), (5, 1020), (2, 1024), (7, 4100), (3, 8192), (2, 16384),
                                    (1024, 4096)])
@pytest.mark.parametrize("mode", [0, 1])
def test_rmsnorm_parity(rows, d, mode):
    announce(f"rmsnorm rows={rows} d={d} mode={mode}")
    x, g = inputs(rows, d, rows + d)
    for eps in (1e-5, 0.0):
        ref = oracle.rmsnorm_f64(x, g, eps)
        y = run(x, g, eps, mode).astype(np.float64)
        err = np.abs(y - ref)
        assert np.all(err <= 4e-6 * np.abs(ref)), (eps, float(np.max(err / (np.abs(ref) + 1e-300))))


def test_zero_rows_give_zero():
    """A zero row with eps > 0 normalises to exactly zero in both forms."""
    x = np.zeros((3, 256), np.float32)
    g = np.ones(256, np.float32)
    for mode in (0, 1):
        assert not run(x, g, 1e-5, mode).any()


def test_many_short_rows():
    """65536 rows of 64 (one workgroup per row, most lanes idle)."""
    announce("rmsnorm 65536 x 64")
    x, g = inputs(65536, 64, 9)
    for mode in (0, 1):
        ref = oracle.rmsnorm_f64(x, g, 1e-5)
        y = run(x, g, 1e-5, mode).astype(np.float64)
        assert np.all(np.abs(y - ref) <= 4e-6 * np.abs(ref)), mode


def test_unfused_on_a_side_stream_without_workspace():
    """The four-pass form on a stream other than torch's current one, with
    the binding allocating its workspace: allocated on that stream, so its
    passes and the caching allocator's reuse are ordered; matches the
    default-stream result bit for bit."""
    announce("rmsnorm unfused, side stream, binding-owned workspace")
    rows, d = 64, 4096
    x, g = inputs(rows, d, 77)
    base = run(x, g, 1e-5, 1)
    xd, gd = torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda()
    side = torch.cuda.Stream()
    for handle in (side, side.cuda_stream):
        yd = torch.empty_like(xd)
        side.wait_stream(torch.cuda.current_stream())
        fc.fc_rmsnorm(xd, gd, yd, 1e-5, 1, None, stream=handle)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert np.array_equal(yd.cpu().numpy(), base)


def random_rmsnorm_shapes():
    rng = np.random.default_rng(20261002 + 3)
    return [(int(rng.integers(1, 300)), 4 * int(rng.integers(1, 4097))) for _ in range(8)]


@pytest.mark.parametrize("rows,d", random_rmsnorm_shapes())
def test_random_shapes_both_forms(rows, d):
    """Seeded random row counts and widths (any multiple of 4 up to 16384):
    both forms against the oracle."""
    announce(f"rmsnorm random shape rows={rows} d={d}")
    x, g = inputs(rows, d, rows * 7 + d)
    ref = oracle.rmsnorm_f64(x, g, 1e-5)
    for mode in (0, 1):
        y = run(x, g, 1e-5, mode).astype(np.float64)
        assert np.all(np.abs(y - ref) <= 4e-6 * np.abs(ref)), mode
