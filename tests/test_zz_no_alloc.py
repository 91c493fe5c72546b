"""The no-allocation GEMM entry point (fc_gemm_epilogue_noalloc) against
fc_gemm_epilogue, the entry point whose kernels it shares: each pair of calls
in a row, the second on a smaller input, gives the same Y bit for bit and
meets the oracle's bar |Y - ref| <= 1e-2 (1 + |ref|) (the chain of "K4 讲解：
fusion 的三笔账", section 1).  The pairs reuse the library's one scratch array
across shapes: a split-K call after a cut plan whose intermediate sat where the
arrival counters go, and the reverse.
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
from gpu_util import f16_from_bits, bits, announce  # noqa: E402


def make(M, N, K, salt):
    h = synth.gemm_inputs(M, N, K, salt)
    return h, [f16_from_bits(t) for t in h]


def both(h, d, plan):
    """Y of the workspace entry point (zero-filled workspace of its own) and of
    the no-allocation one, as fp16 bits."""
    M, K = h[0].shape
    N = h[1].shape[1]
    Y0 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    fc.fc_gemm_epilogue(*d, Y0, plan)
    Y1 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    fc.fc_gemm_epilogue_noalloc(*d, Y1, plan)
    torch.cuda.synchronize()
    return bits(Y0), bits(Y1)


def within_bar(y_bits, ref):
    y = y_bits.view(np.float16).astype(np.float64)
    return float(np.max(np.abs(y - ref) / (1e-2 * (1.0 + np.abs(ref)))))


# (first call, second call on a smaller input): shape (M, N, K) and plan
PAIRS = [
    (((16, 4096, 4096), [1, 3]), ((16, 2048, 2048), [4])),        # decode split-K, then a smaller split
    (((2048, 4096, 1024), [2, 2]), ((200, 2048, 2048), [4])),     # 16 MiB intermediate, then 128x128 split-K
    (((200, 2048, 2048), [1, 1, 2]), ((64, 1024, 1024), [1, 3])), # split-K with cuts, then decode with a cut
    (((4096, 4096, 512), [1, 1, 1, 1]), ((300, 520, 1000), [3, 1])),  # 32 MiB intermediate, then a small mid shape
]


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_workspace_entry_point(pair):
    for step, ((M, N, K), plan) in enumerate(PAIRS[pair]):
        announce(f"gemm noalloc pair {pair} call {step}: {M}x{N}x{K} plan={plan}")
        assert fc.fc_gemm_workspace_bytes(M, N, K, plan) <= fc.FC_GEMM_NOALLOC_SCRATCH_BYTES
        h, d = make(M, N, K, salt=900 + 10 * pair + step)
        y0, y1 = both(h, d, plan)
        assert np.array_equal(y0, y1), (pair, step, int(np.count_nonzero(y0 != y1)))
        ref = oracle.gemm_epilogue_f64_matmul(*h)
        assert within_bar(y1, ref) <= 1.0


def test_noalloc_repeated_calls_same_result():
    """Twelve back-to-back calls alternating two input sets of a split-K shape
    give the first result of each set bit for bit (the counters are cleared on
    every call, stale partials are never read)."""
    M, N, K = 16, 4096, 4096
    announce("gemm noalloc twelve calls")
    sets = [make(M, N, K, salt=s) for s in (951, 952)]
    outs = []
    for it in range(12):
        h, d = sets[it % 2]
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        fc.fc_gemm_epilogue_noalloc(*d, Y, [4])
        outs.append(Y)
    torch.cuda.synchronize()
    outs = [bits(y) for y in outs]
    for it, y in enumerate(outs):
        assert np.array_equal(y, outs[it % 2]), it
    for k in range(2):
        ref = oracle.gemm_epilogue_f64_matmul(*sets[k][0])
        assert within_bar(outs[k], ref) <= 1.0


def test_noalloc_rejects_what_exceeds_its_scratch():
    """A call whose scratch need exceeds the fixed array returns FC_ERR_SCRATCH
    before launching anything (Y untouched); the same shape without a cut,
    which needs no scratch, runs."""
    M, N, K = 4096, 8256, 64                      # a cut needs 2*M*N > 64 MiB
    announce("gemm noalloc over the limit")
    assert fc.fc_gemm_workspace_bytes(M, N, K, [1, 3]) > fc.FC_GEMM_NOALLOC_SCRATCH_BYTES
    h, d = make(M, N, K, salt=960)
    Y = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    with pytest.raises(fc.FcError) as e:
        fc.fc_gemm_epilogue_noalloc(*d, Y, [1, 3])
    assert e.value.status == fc.FC_ERR_SCRATCH
    torch.cuda.synchronize()
    assert not bool(Y.any())
    fc.fc_gemm_epilogue_noalloc(*d, Y, [4])
    torch.cuda.synchronize()
    ref = oracle.gemm_epilogue_f64_matmul(*h)
    assert within_bar(bits(Y), ref) <= 1.0


def test_noalloc_captured_in_a_graph():
    """The callers it is for: two calls (a split-K decode shape with a cut,
    then a split-K 128x128-ring shape) captured in one HIP graph on torch's
    capture stream and replayed four times, with eager work and synchronisation
    between the replays: every replay gives the eager result bit for bit (the
    arrival counters are cleared by a kernel, so the graph holds no memset)."""
    announce("gemm noalloc captured in a graph")
    calls = [((16, 4096, 4096), [1, 3], 970), ((200, 2048, 2048), [4], 971)]
    data = []
    for (M, N, K), plan, salt in calls:
        h, d = make(M, N, K, salt)
        data.append((h, d, plan, torch.empty((M, N), dtype=torch.float16, device="cuda")))

    def work():
        for _, d, plan, Y in data:
            fc.fc_gemm_epilogue_noalloc(*d, Y, plan)

    work()
    torch.cuda.synchronize()
    eager = [bits(Y) for _, _, _, Y in data]
    for (h, _, _, _), y in zip(data, eager):
        assert within_bar(y, oracle.gemm_epilogue_f64_matmul(*h)) <= 1.0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        for _, _, _, Y in data:
            Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (_, _, _, Y) in enumerate(data):
            assert np.array_equal(bits(Y), eager[i]), (rep, i)
