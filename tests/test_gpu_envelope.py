"""The measurement probes of libfcenv.so move exactly the data their header
describes (they are timed beside the hot-path kernels as reachable ceilings,
so they must do the stated work and no less)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gemm_epilogues_amd import envelope as env  # noqa: E402
from gpu_util import announce  # noqa: E402

C = 32768


def test_copy_and_mixed_streams():
    announce("envelope stream probes")
    dev = torch.device("cuda", 0)
    wc, rc = 40, 13
    src = torch.randint(-2**31, 2**31 - 1, (wc * C // 4,), dtype=torch.int32, device=dev)
    dst = torch.zeros_like(src)
    env.fce_mix(src, wc * C, dst, wc * C)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)                     # read == write: a plain copy
    env.fce_mix(src, rc * C, dst, wc * C)
    torch.cuda.synchronize()
    s = src.view(torch.float32).cpu().numpy().reshape(-1, C // 4)
    d = dst.view(torch.float32).cpu().numpy().reshape(-1, C // 4)
    const = np.tile(np.stack([np.full(256, 1.0), np.full(256, 2.0), np.full(256, 3.0),
                              np.arange(256, dtype=np.float64)], 1).reshape(-1), 8).astype(np.float32)
    owners = 0
    for w in range(wc):
        r0, r1 = w * rc // wc, (w + 1) * rc // wc
        if r1 > r0:
            owners += 1
            assert np.array_equal(d[w].view(np.int32), s[r0].view(np.int32)), w
        else:
            assert np.array_equal(d[w], const), w
    assert owners == rc
    env.fce_mix(None, 0, dst, wc * C)                # pure write
    torch.cuda.synchronize()
    assert all(np.array_equal(r, const) for r in dst.view(torch.float32).cpu().numpy().reshape(-1, C // 4))


def test_read_and_mfma_probes_run():
    announce("envelope read and MFMA probes")
    dev = torch.device("cuda", 0)
    src = torch.randn(8 * C // 4, device=dev)
    sink = torch.full((1,), 7.0, device=dev)
    env.fce_read(src, 8 * C, sink)
    msink = torch.empty(env.fce_mfma_sink_floats(), device=dev)
    env.fce_mfma(msink, 4)
    a = msink.clone()
    env.fce_mfma(msink, 4)
    torch.cuda.synchronize()
    assert sink.item() == 7.0
    assert torch.isfinite(msink).all() and torch.equal(a, msink) and msink.abs().sum() > 0


def test_flat_streams():
    """fce_flat copies src to dst exactly, or writes its constant pattern
    (1, 2, 3, lane) per 16 bytes over the whole buffer."""
    announce("envelope flat streams")
    dev = torch.device("cuda", 0)
    nbytes = 37 * 4096
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
    dst = torch.zeros_like(src)
    env.fce_flat(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    env.fce_flat(None, dst, nbytes)
    torch.cuda.synchronize()
    d = dst.view(torch.float32).cpu().numpy().reshape(-1, 4)
    lane = np.arange(d.shape[0]) % 256
    assert np.array_equal(d, np.stack([np.full(lane.size, 1.0), np.full(lane.size, 2.0), np.full(lane.size, 3.0),
                                       lane.astype(np.float64)], 1).astype(np.float32))


def test_repeated_launch_probes():
    """fce_mix_n and fce_empty_n launch their kernel n times: a copy repeated
    three times leaves the plain copy, and a mixed stream the same bytes as
    one call."""
    announce("envelope repeated launches")
    dev = torch.device("cuda", 0)
    wc, rc = 24, 7
    src = torch.randint(-2**31, 2**31 - 1, (wc * C // 4,), dtype=torch.int32, device=dev)
    dst, dst1 = torch.zeros_like(src), torch.zeros_like(src)
    env.fce_mix_n(src, wc * C, dst, wc * C, 3)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    env.fce_mix(src, rc * C, dst1, wc * C)
    env.fce_mix_n(src, rc * C, dst, wc * C, 5)
    torch.cuda.synchronize()
    assert torch.equal(dst, dst1)
    sink = torch.full((1,), 3.0, device=dev)
    env.fce_empty_n(256, 50, sink)
    torch.cuda.synchronize()
    assert sink.item() == 3.0
