"""Python binding of the fused-chain library (libfc.so, C ABI in include/fc.h).

Argument marshalling only: every function here checks tensor dtypes/devices,
passes raw device pointers and the current HIP stream to the C entry point of
the same name, and raises FcError on a non-zero status.  All arithmetic runs
in the HIP kernels.  Importing fails loudly when the library is not built.

torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfc.so")
ROOT = os.path.dirname(HERE)
HEADER = os.path.join(ROOT, "include", "fc.h")

FC_OK = 0
FC_ERR_NULL = -1
FC_ERR_SHAPE = -2
FC_ERR_ALIGN = -3
FC_ERR_PLAN = -4
FC_ERR_UNSUPPORTED = -5
FC_ERR_WORKSPACE = -6
FC_ERR_HIP = -7
FC_ERR_ALIAS = -8
FC_ERR_SCRATCH = -9

FC_CHAIN_NAIVE = 0
FC_CHAIN_FUSED = 1
FC_CHAIN_FAT = 2
FC_SOFTMAX_FUSED = 0
FC_SOFTMAX_UNFUSED = 1
FC_RMSNORM_FUSED = 0
FC_RMSNORM_UNFUSED = 1
FC_CHAIN_MAX_STAGES = 32

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python gemm_epilogues_amd/build.py` "
                      "(or __graft_entry__.build()) first")

# torch ships its own HIP runtime with the same SONAME (libamdhip64.so.7) as
# ROCm's.  Loading torch first makes libfc.so bind to that same runtime, so the
# stream handles and device pointers torch hands out are valid in our calls.
import torch as _torch_for_runtime  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


_RUNTIMES = _hip_runtimes_mapped()
if len(_RUNTIMES) > 1:
    raise ImportError(f"two HIP runtimes are mapped into this process: {sorted(_RUNTIMES)}")

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_U64 = ctypes.c_uint64
_F = ctypes.c_float

class FcStage(ctypes.Structure):
    _fields_ = [("writes", ctypes.c_double), ("ext_reads", ctypes.c_double), ("flops", ctypes.c_double),
                ("live_regs", ctypes.c_int)]


FC_COST_MAX_LEVELS = 8
FC_COST_MAX_STAGES = 16


class FcCostModel(ctypes.Structure):
    _fields_ = [("hbm_bytes_per_s", ctypes.c_double), ("flops_per_s", ctypes.c_double),
                ("launch_s", ctypes.c_double), ("n_levels", ctypes.c_int),
                ("reg_level", ctypes.c_int * FC_COST_MAX_LEVELS),
                ("mem_factor", ctypes.c_double * FC_COST_MAX_LEVELS), ("spill_factor", ctypes.c_double)]


_SIGS = {
    "fc_chain": (_I, [_P, _P, _I64, _P, _P, _I, _I, _I, _P, _I, _P]),
    "fc_chain_scratch_floats": (_SZ, [_I64, _I, _I, _I]),
    "fc_gemm_epilogue": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _P, _SZ, _P]),
    "fc_gemm_workspace_bytes": (_SZ, [_I, _I, _I, _P, _I]),
    "fc_gemm_epilogue_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _P]),
    "fc_causal_softmax": (_I, [_P, _P, _I64, _I, _F, _I, _I, _P, _SZ, _P]),
    "fc_causal_softmax_f32out": (_I, [_P, _P, _I64, _I, _F, _I, _P]),
    "fc_causal_softmax_tiles": (_I, [_P, _P, _P, _I64, _I, _F, _I, _P]),
    "fc_causal_mask_materialise": (_I, [_P, _I64, _I, _P]),
    "fc_softmax_workspace_bytes": (_SZ, [_I64, _I, _I]),
    "fc_plan_bytes": (_U64, [_I64, _I64, _I64, _P, _I, _I]),
    "fc_plan_launches": (_I, [_P, _I]),
    "fc_chain_bytes": (_U64, [_I64, _I, _I]),
    "fc_softmax_bytes": (_U64, [_I64, _I, _I, _I]),
    "fc_causal_attention": (_I, [_P, _P, _P, _P, _I64, _I, _I, _F, _P]),
    "fc_attention_flops": (_U64, [_I64, _I, _I]),
    "fc_attention_bytes": (_U64, [_I64, _I, _I]),
    "fc_rmsnorm": (_I, [_P, _P, _P, _I64, _I, _F, _I, _P, _SZ, _P]),
    "fc_rmsnorm_workspace_bytes": (_SZ, [_I64, _I, _I]),
    "fc_rmsnorm_bytes": (_U64, [_I64, _I, _I]),
    "fc_segments_time": (ctypes.c_double, [_P, _I, _P, _I, _I, _P]),
    "fc_best_split": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "fc_gemm_epilogue_stages": (_I, [_I64, _I64, _I64, _P]),
    "fc_kernel_info": (_I, [ctypes.c_char_p] + [ctypes.POINTER(_I)] * 6),
    "fc_kernel_name": (ctypes.c_char_p, [_I]),
    "fc_status_string": (ctypes.c_char_p, [_I]),
    "fc_version": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class FcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fc_status_string(status)} ({status})")


def lib():
    return _lib


def fc_status_string(status: int) -> str:
    return _lib.fc_status_string(int(status)).decode()


def fc_version() -> str:
    return _lib.fc_version().decode()


def _check(rc: int, where: str) -> None:
    if rc != FC_OK:
        raise FcError(rc, where)


# ---------------------------------------------------------------- marshalling helpers

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    """Raw address of a tensor (or an int address, or None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        torch = _torch()
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call_workspace(nbytes: int, device, stream, zero: bool):
    """A workspace the binding owns for one call.  It is allocated (and
    zero-filled) on the launch stream, so the fill is ordered before the
    kernels and torch's caching allocator hands the block out again only to
    later work on that same stream."""
    torch = _torch()
    if stream is None:
        s = torch.cuda.current_stream(device)
    elif isinstance(stream, int):
        s = torch.cuda.ExternalStream(stream, device=device)
    else:
        s = stream
    with torch.cuda.stream(s):
        return (torch.zeros if zero else torch.empty)(nbytes, dtype=torch.uint8, device=device)


def _dev(t, dtype, name):
    torch = _torch()
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _int_array(seq: Sequence[int]):
    arr = (ctypes.c_int * max(1, len(seq)))(*[int(v) for v in seq])
    return arr, len(seq)


def _f32_array(seq):
    a = np.ascontiguousarray(np.asarray(seq, dtype=np.float32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- chain

def fc_chain_scratch_floats(n: int, K: int, mode: int, fat_temps: int = 0) -> int:
    return int(_lib.fc_chain_scratch_floats(int(n), int(K), int(mode), int(fat_temps)))


def fc_chain(x, y, a, b, relu_even: bool = True, mode: int = FC_CHAIN_FUSED, scratch=None,
             fat_temps: int = 0, stream=None) -> None:
    """y = chain(x); x, y fp32 device tensors of equal size; a, b host sequences."""
    torch = _torch()
    _dev(x, torch.float32, "x")
    _dev(y, torch.float32, "y")
    _dev(scratch, torch.float32, "scratch")
    if x.numel() != y.numel():
        raise ValueError("x and y differ in size")
    av, ap = _f32_array(a)
    bv, bp = _f32_array(b)
    if av.size != bv.size:
        raise ValueError("a and b differ in length")
    if scratch is not None and scratch.numel() < fc_chain_scratch_floats(x.numel(), av.size, mode, fat_temps):
        raise ValueError("scratch too small")
    rc = _lib.fc_chain(_ptr(x), _ptr(y), x.numel(), ap, bp, av.size, int(bool(relu_even)),
                       int(mode), _ptr(scratch), int(fat_temps), _stream(stream))
    _check(rc, "fc_chain")


# ---------------------------------------------------------------- GEMM + epilogue

def fc_gemm_workspace_bytes(M: int, N: int, K: int, plan: Sequence[int]) -> int:
    arr, n = _int_array(plan)
    return int(_lib.fc_gemm_workspace_bytes(int(M), int(N), int(K), arr, n))


def fc_gemm_epilogue(A, B, bias, R, Y, plan: Sequence[int], workspace=None, stream=None) -> None:
    """Y = GELU(A@B + bias) + R, fp16 device tensors A [M,K], B [K,N], bias [N], R/Y [M,N].

    A caller-supplied workspace must be zero-filled before its first use (see
    fc_gemm_workspace_bytes); without one, a zero-filled one is allocated on
    the launch stream for this call."""
    torch = _torch()
    for t, nm in ((A, "A"), (B, "B"), (bias, "bias"), (R, "R"), (Y, "Y")):
        _dev(t, torch.float16, nm)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    K2, N = B.shape
    if K != K2 or bias.numel() != N or R.numel() != M * N or Y.numel() != M * N:
        raise ValueError("shape mismatch")
    arr, n = _int_array(plan)
    ws_bytes = 0
    if workspace is None:
        need = int(_lib.fc_gemm_workspace_bytes(M, N, K, arr, n))
        if need:
            # zero-filled, as the split kernels' arrival counters require
            workspace = _call_workspace(need, A.device, stream, zero=True)
    if workspace is not None:
        if not workspace.is_cuda:
            raise ValueError("workspace must be a device tensor")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.fc_gemm_epilogue(_ptr(A), _ptr(B), _ptr(bias), _ptr(R), _ptr(Y), M, N, K, arr, n,
                               _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "fc_gemm_epilogue")


# fixed scratch of fc_gemm_epilogue_noalloc (FC_GEMM_NOALLOC_SCRATCH_BYTES in fc.h)
FC_GEMM_NOALLOC_SCRATCH_BYTES = 64 << 20


def fc_gemm_epilogue_noalloc(A, B, bias, R, Y, plan: Sequence[int], stream=None) -> None:
    """fc_gemm_epilogue through the entry point that allocates nothing: the
    library's own fixed per-device scratch holds the split-K partials and the
    cut intermediate (calls needing more than FC_GEMM_NOALLOC_SCRATCH_BYTES
    raise FcError(FC_ERR_SCRATCH)).  Calls that overlap in time on one device race."""
    torch = _torch()
    for t, nm in ((A, "A"), (B, "B"), (bias, "bias"), (R, "R"), (Y, "Y")):
        _dev(t, torch.float16, nm)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    K2, N = B.shape
    if K != K2 or bias.numel() != N or R.numel() != M * N or Y.numel() != M * N:
        raise ValueError("shape mismatch")
    arr, n = _int_array(plan)
    rc = _lib.fc_gemm_epilogue_noalloc(_ptr(A), _ptr(B), _ptr(bias), _ptr(R), _ptr(Y), M, N, K, arr, n,
                                       _stream(stream))
    _check(rc, "fc_gemm_epilogue_noalloc")


# ---------------------------------------------------------------- causal softmax

def fc_softmax_workspace_bytes(BH: int, S: int, mode: int) -> int:
    return int(_lib.fc_softmax_workspace_bytes(int(BH), int(S), int(mode)))


def _bhs(scores):
    if scores.dim() == 3:
        BH, S, S2 = scores.shape
    elif scores.dim() == 4:
        B, H, S, S2 = scores.shape
        BH = B * H
    else:
        raise ValueError("scores must be [BH,S,S] or [B,H,S,S]")
    if S != S2:
        raise ValueError("scores must be square in the last two dims")
    return BH, S


def fc_causal_softmax(scores, out, scale: float, tile: int, mode: int = FC_SOFTMAX_FUSED,
                      workspace=None, stream=None) -> None:
    """out = causal softmax(scale * scores); bf16 device tensors [BH,S,S] or [B,H,S,S]."""
    torch = _torch()
    _dev(scores, torch.bfloat16, "scores")
    _dev(out, torch.bfloat16, "out")
    BH, S = _bhs(scores)
    if out.numel() != scores.numel():
        raise ValueError("out size mismatch")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.fc_causal_softmax(_ptr(scores), _ptr(out), BH, S, float(scale), int(tile), int(mode),
                                _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "fc_causal_softmax")


def fc_causal_softmax_f32out(scores, out, scale: float, tile: int, stream=None) -> None:
    torch = _torch()
    _dev(scores, torch.bfloat16, "scores")
    _dev(out, torch.float32, "out")
    BH, S = _bhs(scores)
    if out.numel() != scores.numel():
        raise ValueError("out size mismatch")
    rc = _lib.fc_causal_softmax_f32out(_ptr(scores), _ptr(out), BH, S, float(scale), int(tile),
                                       _stream(stream))
    _check(rc, "fc_causal_softmax_f32out")


def fc_causal_softmax_tiles(scores, out, tiles_per_row, scale: float, tile: int, stream=None) -> None:
    torch = _torch()
    _dev(scores, torch.bfloat16, "scores")
    _dev(out, torch.bfloat16, "out")
    _dev(tiles_per_row, torch.int32, "tiles_per_row")
    BH, S = _bhs(scores)
    if tiles_per_row.numel() != BH * S:
        raise ValueError("tiles_per_row must have BH*S entries")
    rc = _lib.fc_causal_softmax_tiles(_ptr(scores), _ptr(out), _ptr(tiles_per_row), BH, S,
                                      float(scale), int(tile), _stream(stream))
    _check(rc, "fc_causal_softmax_tiles")


def fc_causal_mask_materialise(mask, BH: int, S: int, stream=None) -> None:
    """mask: a bf16 device tensor of >= BH*S*S elements, or a device address."""
    if not isinstance(mask, int):
        torch = _torch()
        if not mask.is_cuda:
            raise ValueError("mask must be a device tensor")
        if mask.numel() * mask.element_size() < 2 * BH * S * S:
            raise ValueError("mask too small")
        if not mask.is_contiguous():
            raise ValueError("mask must be contiguous")
        del torch
    rc = _lib.fc_causal_mask_materialise(_ptr(mask), int(BH), int(S), _stream(stream))
    _check(rc, "fc_causal_mask_materialise")


# ---------------------------------------------------------------- causal attention

def fc_causal_attention(Q, K, V, O, scale: float, stream=None) -> None:
    """O = causal softmax(scale * Q K^T) V; bf16 device tensors [BH, S, D] or [B, H, S, D]."""
    torch = _torch()
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V"), (O, "O")):
        _dev(t, torch.bfloat16, nm)
    if Q.dim() not in (3, 4) or not (Q.shape == K.shape == V.shape == O.shape):
        raise ValueError("Q, K, V, O must share one [BH,S,D] or [B,H,S,D] shape")
    S, D = Q.shape[-2], Q.shape[-1]
    BH = Q.numel() // (S * D) if S * D else 0
    rc = _lib.fc_causal_attention(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), int(BH), int(S), int(D),
                                  float(scale), _stream(stream))
    _check(rc, "fc_causal_attention")


def fc_attention_flops(BH: int, S: int, D: int) -> int:
    return int(_lib.fc_attention_flops(int(BH), int(S), int(D)))


def fc_attention_bytes(BH: int, S: int, D: int) -> int:
    return int(_lib.fc_attention_bytes(int(BH), int(S), int(D)))


# ---------------------------------------------------------------- RMSNorm

def fc_rmsnorm_workspace_bytes(rows: int, d: int, mode: int) -> int:
    return int(_lib.fc_rmsnorm_workspace_bytes(int(rows), int(d), int(mode)))


def fc_rmsnorm_bytes(rows: int, d: int, mode: int) -> int:
    return int(_lib.fc_rmsnorm_bytes(int(rows), int(d), int(mode)))


def fc_rmsnorm(x, g, y, eps: float, mode: int = FC_RMSNORM_FUSED, workspace=None, stream=None) -> None:
    """y = x / sqrt(mean(x^2, row) + eps) * g; fp32 device tensors x, y [rows, d], g [d]."""
    torch = _torch()
    for t, nm in ((x, "x"), (g, "g"), (y, "y")):
        _dev(t, torch.float32, nm)
    if x.dim() != 2 or y.shape != x.shape or g.numel() != x.shape[1]:
        raise ValueError("x, y must be [rows, d] and g [d]")
    rows, d = x.shape
    ws_bytes = 0
    if workspace is None and mode == FC_RMSNORM_UNFUSED:
        need = fc_rmsnorm_workspace_bytes(rows, d, mode)
        if need:
            workspace = _call_workspace(need, x.device, stream, zero=False)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.fc_rmsnorm(_ptr(x), _ptr(g), _ptr(y), int(rows), int(d), float(eps), int(mode),
                         _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "fc_rmsnorm")


# ---------------------------------------------------------------- cost model (host only)

def cost_model(hbm_bytes_per_s: float, flops_per_s: float, launch_s: float,
               levels=((255, 1.0),), spill_factor: float = 3.0) -> FcCostModel:
    """Model parameters; `levels` are (register level, memory-time factor) pairs
    in increasing register order.  Defaults follow the pages' single 255
    threshold with factor 3 beyond it."""
    m = FcCostModel()
    m.hbm_bytes_per_s, m.flops_per_s, m.launch_s = float(hbm_bytes_per_s), float(flops_per_s), float(launch_s)
    m.n_levels = len(levels)
    for i, (r, f) in enumerate(levels):
        m.reg_level[i], m.mem_factor[i] = int(r), float(f)
    m.spill_factor = float(spill_factor)
    return m


def _stages(stages):
    arr = (FcStage * len(stages))()
    for i, st in enumerate(stages):
        arr[i] = st if isinstance(st, FcStage) else FcStage(*st)
    return arr, len(stages)


def fc_gemm_epilogue_stages(M: int, N: int, K: int):
    arr = (FcStage * 4)()
    _check(_lib.fc_gemm_epilogue_stages(int(M), int(N), int(K), arr), "fc_gemm_epilogue_stages")
    return [arr[i] for i in range(4)]


def fc_segments_time(stages, plan: Sequence[int], elem_bytes: int, model: FcCostModel) -> float:
    arr, n = _stages(stages)
    parr, pn = _int_array(plan)
    return float(_lib.fc_segments_time(arr, n, parr, pn, int(elem_bytes), ctypes.byref(model)))


def fc_best_split(stages, elem_bytes: int, model: FcCostModel):
    """(plan, estimated seconds) with the least estimate over all compositions."""
    arr, n = _stages(stages)
    out = (ctypes.c_int * FC_COST_MAX_STAGES)()
    ln, t = ctypes.c_int(0), ctypes.c_double(0.0)
    _check(_lib.fc_best_split(arr, n, int(elem_bytes), ctypes.byref(model), out, ctypes.byref(ln),
                              ctypes.byref(t)), "fc_best_split")
    return [out[i] for i in range(ln.value)], t.value


# ---------------------------------------------------------------- accounting (host only)

def fc_plan_bytes(M: int, N: int, K: int, plan: Sequence[int], elem_bytes: int = 2) -> int:
    arr, n = _int_array(plan)
    return int(_lib.fc_plan_bytes(int(M), int(N), int(K), arr, n, int(elem_bytes)))


def fc_plan_launches(plan: Sequence[int]) -> int:
    arr, n = _int_array(plan)
    return int(_lib.fc_plan_launches(arr, n))


def fc_chain_bytes(n: int, K: int, mode: int) -> int:
    return int(_lib.fc_chain_bytes(int(n), int(K), int(mode)))


def fc_softmax_bytes(BH: int, S: int, tile: int, mode: int) -> int:
    return int(_lib.fc_softmax_bytes(int(BH), int(S), int(tile), int(mode)))


# ---------------------------------------------------------------- kernel resources (host only)

KERNEL_INFO_FIELDS = ("vgprs", "agprs", "sgprs", "lds_bytes", "scratch_bytes", "waves_per_simd")


def fc_kernel_info(name: str) -> dict:
    """Compiler resource report of one kernel of the library, by demangled name."""
    vals = [ctypes.c_int(-1) for _ in KERNEL_INFO_FIELDS]
    _check(_lib.fc_kernel_info(name.encode(), *[ctypes.byref(v) for v in vals]), f"fc_kernel_info({name!r})")
    return {f: v.value for f, v in zip(KERNEL_INFO_FIELDS, vals)}


def fc_kernel_names() -> list:
    """Every kernel name fc_kernel_info accepts, in table order."""
    out, i = [], 0
    while True:
        n = _lib.fc_kernel_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1
