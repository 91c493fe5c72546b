"""GPU parity of the fp16 GEMM + bias + erf-GELU + residual chain for every
split plan ("K4 讲解：fusion 的三笔账", section 1) against the fp64 oracle.

Bar: |Y - ref| <= 1e-2 * (1 + |ref|) elementwise for every plan; the GEMM
alone is bit-exact on integer-valued inputs.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import ledger

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gemm_epilogues_amd as fc  # noqa: E402
from gpu_util import f16_from_bits, bits, announce  # noqa: E402

ALL_PLANS = ledger.compositions(4)
NAMED_PLANS = [[1, 1, 1, 1], [1, 3], [2, 2], [4]]


def tol_ok(y_bits, ref):
    y = y_bits.view(np.float16).astype(np.float64)
    err = np.abs(y - ref)
    bound = 1e-2 * (1.0 + np.abs(ref))
    return bool(np.all(err <= bound)), float(np.max(err / bound))


class Dev:
    def __init__(self, M, N, K, salt=0, int_valued=False):
        self.M, self.N, self.K = M, N, K
        if int_valued:
            A, B = synth.gemm_int_inputs(M, N, K, salt)
            _, _, bias, R = synth.gemm_inputs(M, N, K, salt)
        else:
            A, B, bias, R = synth.gemm_inputs(M, N, K, salt)
        self.h = (A, B, bias, R)
        self.A, self.B, self.bias, self.R = (f16_from_bits(t) for t in self.h)

    def run(self, plan, keep_ws=False):
        Y = torch.empty((self.M, self.N), dtype=torch.float16, device="cuda")
        wsb = fc.fc_gemm_workspace_bytes(self.M, self.N, self.K, plan)
        # zero-filled: the decode kernel's arrival counters live here
        ws = torch.zeros(max(wsb // 2, 1), dtype=torch.float16, device="cuda") if wsb else None
        fc.fc_gemm_epilogue(self.A, self.B, self.bias, self.R, Y, plan, ws)
        torch.cuda.synchronize()
        if keep_ws:
            # the intermediate follows the decode scratch, whose size is plan [4]'s workspace
            off = fc.fc_gemm_workspace_bytes(self.M, self.N, self.K, [4]) // 2
            return bits(Y), (bits(ws)[off: off + self.M * self.N].reshape(self.M, self.N)
                             if ws is not None else None)
        return bits(Y)


def check_every_output(d, plans):
    """Every output of every plan against the full fp64 reference (product by
    numpy's fp64 matmul, epilogue by the C oracle), compared on the device."""
    ref = torch.from_numpy(oracle.gemm_epilogue_f64_matmul(*d.h)).cuda()
    bound = 1e-2 * (1.0 + ref.abs())
    for plan in plans:
        Y = torch.empty((d.M, d.N), dtype=torch.float16, device="cuda")
        wsb = fc.fc_gemm_workspace_bytes(d.M, d.N, d.K, plan)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None
        fc.fc_gemm_epilogue(d.A, d.B, d.bias, d.R, Y, plan, ws)
        torch.cuda.synchronize()
        worst = float(((Y.double() - ref).abs() / bound).max())
        assert worst <= 1.0, (plan, worst)


SMALL = [(1, 8, 8), (3, 16, 40), (16, 64, 64), (17, 40, 24), (33, 72, 136), (64, 128, 256),
         (100, 264, 520), (129, 136, 72), (256, 256, 64), (300, 520, 1000)]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_all_plans_small_shapes(M, N, K):
    announce(f"gemm M={M} N={N} K={K} all plans")
    d = Dev(M, N, K, salt=M + N + K)
    ref = oracle.gemm_epilogue_f64(*d.h)
    for plan in ALL_PLANS:
        ok, worst = tol_ok(d.run(plan), ref)
        assert ok, (plan, worst)


def test_big_tile_path_all_plans():
    """Shapes that take the 256x256 tile kernel (>= 128 tiles), with ragged M:
    every output of every plan."""
    M, N, K = 2048 + 37, 4096, 264
    announce(f"gemm big tiles M={M} N={N} K={K}")
    check_every_output(Dev(M, N, K, salt=5), ALL_PLANS)


@pytest.mark.parametrize("M", [1, 16, 17, 64, 256, 4096])
def test_integer_gemm_exact_in_workspace(M):
    """A, B in {-1,0,1}: plan [1,3] leaves C = A.B (fp16) in the workspace,
    bit-exact against the integer product."""
    N, K = (4096, 1024) if M == 4096 else (2048, 2048)
    announce(f"gemm integer exact M={M} N={N} K={K}")
    d = Dev(M, N, K, salt=M, int_valued=True)
    _, C = d.run([1, 3], keep_ws=True)
    A = d.h[0].view(np.float16).astype(np.float64)
    B = d.h[1].view(np.float16).astype(np.float64)
    exact = A @ B            # integer sums of magnitude <= K: exact in fp64
    assert np.array_equal(C.view(np.float16).astype(np.float64), exact)


def test_decode_config_all_plans():
    """M = 16, N = K = 4096 (decode shape), every plan against the full oracle."""
    announce("gemm decode 16x4096x4096")
    d = Dev(16, 4096, 4096)
    ref = oracle.gemm_epilogue_f64(*d.h)
    outs = {}
    for plan in ALL_PLANS:
        Y = d.run(plan)
        ok, worst = tol_ok(Y, ref)
        assert ok, (plan, worst)
        outs[tuple(plan)] = Y
    # the fused plan's only rounding is the final one
    y4 = outs[(4,)].view(np.float16).astype(np.float64)
    assert np.max(np.abs(y4 - ref) / (1 + np.abs(ref))) <= 2.0 ** -10


@pytest.fixture(scope="module")
def square_4096():
    """The 4096^3 workload and its full fp64 reference, computed once (the
    product step by numpy's fp64 matmul, the epilogue by the C oracle)."""
    announce("gemm 4096^3: generating inputs and the full fp64 reference")
    d = Dev(4096, 4096, 4096)
    ref = torch.from_numpy(oracle.gemm_epilogue_f64_matmul(*d.h)).cuda()
    return d, ref


def test_square_4096_config_every_output(square_4096):
    """M = N = K = 4096, all eight split plans: every output within
    1e-2 (1 + |ref|) of the fp64 oracle (compared on the device in fp64), and
    the fused plan, whose only rounding is the final one, within 2^-10."""
    d, ref = square_4096
    bound = 1e-2 * (1.0 + ref.abs())
    for plan in ALL_PLANS:
        announce(f"gemm 4096^3 plan={plan} every output")
        Y = torch.empty((4096, 4096), dtype=torch.float16, device="cuda")
        wsb = fc.fc_gemm_workspace_bytes(4096, 4096, 4096, plan)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda") if wsb else None
        fc.fc_gemm_epilogue(d.A, d.B, d.bias, d.R, Y, plan, ws)
        torch.cuda.synchronize()
        err = (Y.double() - ref).abs()
        worst = float((err / bound).max())
        assert worst <= 1.0, (plan, worst)
        if plan == [4]:
            assert float((err / (1.0 + ref.abs())).max()) <= 2.0 ** -10
        del Y, ws, err


@pytest.mark.parametrize("M,N,K", [(1000, 2000, 320), (2085, 4136, 320), (3109, 4136, 320),
                                   (4096 + 200, 4096 - 8, 192)])
def test_ring_path_ragged_all_plans(M, N, K):
    """K % 64 == 0 with M and N tails (clamped rows/columns are computed but
    never stored): 128 tiles of 128x128 (one round) take the 128x128 ring
    kernel unsplit; 561, 825 and 1088 take the 256x256 one.  Every output."""
    announce(f"gemm ring path M={M} N={N} K={K}")
    check_every_output(Dev(M, N, K, salt=11), ALL_PLANS)


@pytest.mark.parametrize("M,N,K", [(16, 4096, 64), (300, 520, 64), (4096, 4096, 64)])
def test_gelu_epilogue_accuracy(M, N, K):
    """A = 0 and R = 0 give Y = fp16(GELU(bias)) exactly up to the final
    rounding: every plan's GELU (fused on the accumulators or pointwise) is
    within one fp16 ulp of the fp64 oracle, for bias spanning [-8, 8]."""
    announce(f"gelu accuracy M={M} N={N} K={K}")
    A = np.zeros((M, K), np.uint16)
    B = synth.gemm_inputs(8, N, K, salt=1)[1]
    zs = np.linspace(-8.0, 8.0, N)
    bias = synth.f64_to_f16_bits(zs)
    R = np.zeros((M, N), np.uint16)
    d = Dev(1, 8, 8)
    d.M, d.N, d.K = M, N, K
    d.h = (A, B, bias, R)
    d.A, d.B, d.bias, d.R = (f16_from_bits(x) for x in d.h)
    ref = oracle.gemm_epilogue_f64(A[:1], B, bias, R[:1])[0]
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    for plan in ALL_PLANS:
        Y = d.run(plan).view(np.float16).astype(np.float64)
        assert np.all(Y == Y[0]), plan
        assert np.all(np.abs(Y[0] - ref) <= ulp + 1e-12), (plan, float(np.max(np.abs(Y[0] - ref) / ulp)))


# Shapes of the split-K decode kernel.  M <= 16 (one 16-row block): no split
# (one or a few workgroups, or 512 strips), 1-, 2- and 4-step waves, P = 2, 4,
# 8, 16 and 64.  17..32 rows (two blocks) and 33..64 rows (four blocks, at
# most 2 k-steps per wave): no split, P = 2, 8, 16 and 32, ragged row counts.
DECODE_SHAPES = [(1, 64, 256), (5, 640, 768), (16, 4096, 1024), (16, 4096, 8192), (1, 2048, 2048),
                 (16, 64, 65536), (7, 16384, 512), (3, 32768, 256),
                 (17, 4096, 4096), (32, 640, 768), (33, 2048, 2048), (64, 4096, 4096), (48, 64, 8192),
                 (64, 16384, 512)]


@pytest.mark.parametrize("M,N,K", DECODE_SHAPES)
def test_decode_kernel_shapes_all_plans(M, N, K):
    announce(f"gemm decode path M={M} N={N} K={K} all plans")
    d = Dev(M, N, K, salt=7 * M + N + K)
    ref = oracle.gemm_epilogue_f64(*d.h)
    for plan in ALL_PLANS:
        ok, worst = tol_ok(d.run(plan), ref)
        assert ok, (plan, worst)


@pytest.mark.parametrize("M", [16, 64])
@pytest.mark.parametrize("plan", [[4], [1, 3]])
def test_decode_workspace_reuse(plan, M):
    """One zero-filled workspace for twelve back-to-back calls on two input
    sets: every result matches the oracle and is bit-identical to the first
    result of its set (the split partials are summed in a fixed order and no
    stale partial from the previous call is read), and the arrival counters
    are zero again afterwards."""
    N, K = 4096, 4096
    announce(f"gemm decode workspace reuse plan={plan} M={M}")
    sets = [Dev(M, N, K, salt=21), Dev(M, N, K, salt=22)]
    refs = [oracle.gemm_epilogue_f64(*d.h) for d in sets]
    wsb = fc.fc_gemm_workspace_bytes(M, N, K, plan)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    Ys = []
    for it in range(12):
        d = sets[it % 2]
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        fc.fc_gemm_epilogue(d.A, d.B, d.bias, d.R, Y, plan, ws)
        Ys.append(Y)
    torch.cuda.synchronize()
    outs = [bits(Y) for Y in Ys]
    for it, y in enumerate(outs):
        ok, worst = tol_ok(y, refs[it % 2])
        assert ok, (it, worst)
        assert np.array_equal(y, outs[it % 2]), it
    counters = ws[: 4 * (N // 64)].cpu().numpy().view(np.uint32)
    assert not counters.any()


def test_decode_workspace_shared_by_plans():
    """All eight plans in turn on one workspace (the counters sit at offset 0
    for every plan of a shape), twice over."""
    M, N, K = 16, 2048, 2048
    announce("gemm decode one workspace for all plans")
    d = Dev(M, N, K, salt=23)
    ref = oracle.gemm_epilogue_f64(*d.h)
    wsb = max(fc.fc_gemm_workspace_bytes(M, N, K, p) for p in ALL_PLANS)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    Ys = []
    for plan in ALL_PLANS + ALL_PLANS:
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        fc.fc_gemm_epilogue(d.A, d.B, d.bias, d.R, Y, plan, ws)
        Ys.append((plan, Y))
    torch.cuda.synchronize()
    for plan, Y in Ys:
        ok, worst = tol_ok(bits(Y), ref)
        assert ok, (plan, worst)


# Shapes with at most 512 tiles of 128x128 and K % 64 == 0 (and beyond the
# decode kernel) run the 128x128 ring kernel, K split P ways when its tiles
# number fewer than 128 (the last workgroup of a tile sums the fp32 partials in
# split order): from 65 rows on, P = 4, 4, 4, 2, 4, 4, 2 and 2, ragged rows
# and columns included.
RING128_SHAPES = [(65, 4096, 4096), (100, 640, 1024), (128, 2048, 2048), (129, 4096, 4096), (300, 1000, 1024),
                  (200, 2048, 2048), (1024, 1024, 1024), (520, 264, 640)]


@pytest.mark.parametrize("M,N,K", RING128_SHAPES)
def test_ring128_shapes_all_plans(M, N, K):
    announce(f"gemm ring128 M={M} N={N} K={K} all plans")
    assert fc.fc_gemm_workspace_bytes(M, N, K, [4]) > 0      # the split path is the one under test
    d = Dev(M, N, K, salt=11 * M + N + K)
    ref = oracle.gemm_epilogue_f64(*d.h)
    for plan in ALL_PLANS:
        ok, worst = tol_ok(d.run(plan), ref)
        assert ok, (plan, worst)


def test_ring128_512_every_output():
    """512 x 4096 x 4096 (128 tiles of 128x128, no split): every output of
    every plan."""
    announce("gemm ring128 512x4096x4096 every output")
    check_every_output(Dev(512, 4096, 4096, salt=5), ALL_PLANS)


def test_ring128_workspace_reuse():
    """One zero-filled workspace for twelve back-to-back calls on two input
    sets of a split shape: every result matches the oracle and equals the
    first result of its set bit for bit, and the tile counters end at zero."""
    M, N, K = 200, 2048, 2048
    announce("gemm ring128 workspace reuse")
    sets = [Dev(M, N, K, salt=31), Dev(M, N, K, salt=32)]
    refs = [oracle.gemm_epilogue_f64(*d.h) for d in sets]
    ws = torch.zeros(fc.fc_gemm_workspace_bytes(M, N, K, [4]), dtype=torch.uint8, device="cuda")
    Ys = []
    for it in range(12):
        d = sets[it % 2]
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        fc.fc_gemm_epilogue(d.A, d.B, d.bias, d.R, Y, [4], ws)
        Ys.append(Y)
    torch.cuda.synchronize()
    outs = [bits(Y) for Y in Ys]
    for it, y in enumerate(outs):
        ok, worst = tol_ok(y, refs[it % 2])
        assert ok, (it, worst)
        assert np.array_equal(y, outs[it % 2]), it
    tiles = ((M + 127) // 128) * ((N + 127) // 128)
    assert not ws[: 4 * tiles].cpu().numpy().view(np.uint32).any()


@pytest.mark.parametrize("M,N,K", [(16, 4096, 4096), (200, 2048, 2048)])
def test_side_stream_without_workspace(M, N, K):
    """No workspace passed and a stream other than torch's current one: the
    binding zero-fills its own workspace on that stream, so the split kernels'
    arrival counters are zero when they run; every plan matches the oracle and
    the default-stream result bit for bit, also with a busy current stream."""
    announce(f"gemm side stream, binding-owned workspace {M}x{N}x{K}")
    d = Dev(M, N, K, salt=31)
    ref = oracle.gemm_epilogue_f64(*d.h)
    side = torch.cuda.Stream()
    for plan in NAMED_PLANS:
        base = d.run(plan)
        outs = []
        for handle in (side, side.cuda_stream):      # a torch stream, then a raw handle
            Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
            # a freed block of the workspace's size full of 0xFF on the current
            # stream, then work left queued there: a workspace taken and filled
            # on the current stream would reach the kernels unfilled
            need = fc.fc_gemm_workspace_bytes(M, N, K, plan)
            dirty = torch.full((max(need, 1),), 255, dtype=torch.uint8, device="cuda")
            del dirty
            side.wait_stream(torch.cuda.current_stream())
            busy = torch.empty(1 << 24, device="cuda").normal_()
            fc.fc_gemm_epilogue(d.A, d.B, d.bias, d.R, Y, plan, None, stream=handle)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            del busy
            outs.append(bits(Y))
        for y in outs:
            ok, worst = tol_ok(y, ref)
            assert ok, (plan, worst)
            assert np.array_equal(y, base), plan


def random_shapes():
    """Seeded shapes for each kernel route: split-K decode (M <= 64, N % 64 = 0,
    K % 256 = 0), the M <= 16 kernel without a decode split (K % 256 != 0),
    the 128x128 ring (K % 64 = 0), the register-staged kernels (K % 64 != 0)
    and the 256x256 ring (more than 512 tiles of 128x128)."""
    rng = np.random.default_rng(20261002)
    out = []
    for _ in range(5):
        out.append((int(rng.integers(1, 65)), 64 * int(rng.integers(1, 20)), 256 * int(rng.integers(1, 5))))
        out.append((int(rng.integers(1, 17)), 8 * int(rng.integers(1, 150)), 8 * int(rng.integers(1, 128)) | 8))
        out.append((int(rng.integers(65, 700)), 8 * int(rng.integers(1, 150)), 64 * int(rng.integers(1, 17))))
        out.append((int(rng.integers(17, 700)), 8 * int(rng.integers(1, 150)), 8 * int(rng.integers(1, 128)) | 8))
    for _ in range(2):
        out.append((int(rng.integers(2049, 2400)), 8 * int(rng.integers(513, 640)), 64 * int(rng.integers(1, 4))))
    return out


@pytest.mark.parametrize("M,N,K", random_shapes())
def test_random_shapes_every_output(M, N, K):
    """Every output of all eight plans against the oracle on seeded random
    shapes that reach every kernel route, ragged edges included."""
    announce(f"gemm random shape {M}x{N}x{K}")
    check_every_output(Dev(M, N, K, salt=M + N + K), ALL_PLANS)
