"""The library's launches captured in a HIP graph and replayed: every replay,
with the program's own eager work and synchronisations between replays, gives
the eager result bit for bit.  Covers each entry point in the modes the
benchmark captures (fused/naive/fat chain, decode-shape GEMM with its arrival
counters, fused and unfused softmax)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gemm_epilogues_amd as fc  # noqa: E402
from gpu_util import f16_from_bits, announce  # noqa: E402


def test_graph_replays_match_eager():
    announce("graph capture and replay of every entry point")
    dev = torch.device("cuda", 0)
    n, K = 1 << 20, 8
    x, a, b = synth.chain_inputs(n, K, salt=31)
    xd = torch.from_numpy(x).to(dev)
    y_f, y_n, y_t = (torch.empty_like(xd) for _ in range(3))
    scratch = torch.empty(fc.fc_chain_scratch_floats(n, K, fc.FC_CHAIN_NAIVE, 0), dtype=torch.float32,
                          device=dev)
    sink = torch.empty(fc.fc_chain_scratch_floats(n, 4, fc.FC_CHAIN_FAT, 48), dtype=torch.float32,
                       device=dev)
    a4, b4 = synth.chain_inputs(1, 4, salt=32)[1:]

    M, N, Kg = 16, 4096, 4096
    A, B, bias, R = (f16_from_bits(t) for t in synth.gemm_inputs(M, N, Kg, salt=33))
    ws = torch.zeros(max(fc.fc_gemm_workspace_bytes(M, N, Kg, p) for p in ([4], [1, 3])),
                     dtype=torch.uint8, device=dev)
    Y4, Y13 = (torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(2))

    BH, S = 4, 256
    s = torch.from_numpy(synth.softmax_inputs(BH, S, salt=34).view(np.int16)).to(dev).view(torch.bfloat16)
    o_f, o_u = (torch.empty_like(s) for _ in range(2))
    smws = torch.empty(fc.fc_softmax_workspace_bytes(BH, S, fc.FC_SOFTMAX_UNFUSED), dtype=torch.uint8,
                       device=dev)
    outs = (y_f, y_n, y_t, Y4, Y13, o_f, o_u)

    def work():
        fc.fc_chain(xd, y_f, a, b, True, fc.FC_CHAIN_FUSED)
        fc.fc_chain(xd, y_n, a, b, True, fc.FC_CHAIN_NAIVE, scratch)
        fc.fc_chain(xd, y_t, a4, b4, True, fc.FC_CHAIN_FAT, sink, 48)
        fc.fc_gemm_epilogue(A, B, bias, R, Y4, [4], ws)
        fc.fc_gemm_epilogue(A, B, bias, R, Y13, [1, 3], ws)
        fc.fc_causal_softmax(s, o_f, 0.125, 64, fc.FC_SOFTMAX_FUSED)
        fc.fc_causal_softmax(s, o_u, 0.125, 64, fc.FC_SOFTMAX_UNFUSED, smws)

    work()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(-1.0)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            as_int = torch.int32 if o.element_size() == 4 else torch.int16
            assert torch.equal(o.view(as_int), e.view(as_int)), (rep, i)
    counters = ws[: 4 * (N // 64)].cpu().numpy().view(np.uint32)
    assert not counters.any()
