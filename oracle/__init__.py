"""CPU oracle for the fused-chain hot path -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product library (``gemm_epilogues_amd``)
never imports it and shares no code with it.

``oracle.c`` holds the plain fp64 definitions (chain, GEMM + bias + GELU +
residual, causal softmax, causal attention, RMSNorm); ``ledger.py`` the byte
and launch ledgers.  This
module builds ``oracle.c`` with gcc and wraps it with ctypes/numpy.

Every function here is pinned by a CPU test against something other than
itself (closed forms, values the pages print, exact rational brute force,
textbook normal-CDF values, numpy's matmul); see tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import ledger  # noqa: F401  (re-exported)

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", "-std=c11", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        D = ctypes.c_double
        sig = {
            "oracle_chain_f64": [P, P, I64, P, P, I, I],
            "oracle_chain_f32fma": [P, P, I64, P, P, I, I],
            "oracle_chain_fat_sink_f64": [P, I64, P, P, I, I, I, I64, P, P],
            "oracle_chain_fat_sink_f32": [P, I64, P, P, I, I, I, I64, P],
            "oracle_epilogue_on_product_f64": [P, P, P, I64, I64, P],
            "oracle_gemm_f64": [P, P, I64, I64, I64, P],
            "oracle_gemm_epilogue_f64": [P, P, P, P, I64, I64, I64, P],
            "oracle_gemm_epilogue_at": [P, P, P, P, I64, I64, I64, P, P, I64, P],
            "oracle_causal_softmax_rows": [P, I64, D, P, I64, P],
            "oracle_causal_softmax_f64": [P, I64, I64, D, P],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = None
        lib.oracle_rmsnorm_f64.argtypes = [P, P, I64, I64, D, P]
        lib.oracle_rmsnorm_f64.restype = None
        lib.oracle_causal_attention_rows.argtypes = [P, P, P, I64, I64, D, P, I64, P]
        lib.oracle_causal_attention_rows.restype = I
        for name, arg in (("oracle_gelu", D), ("oracle_half_to_double", ctypes.c_uint16),
                          ("oracle_bf16_to_double", ctypes.c_uint16)):
            fn = getattr(lib, name)
            fn.argtypes = [arg]
            fn.restype = D
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- chain

def chain_f64(x, a, b, relu_even: bool = True) -> np.ndarray:
    """y = chain(x) in fp64 ("C-05" section 3 stage operation)."""
    x, a, b = _c(x, np.float32), _c(a, np.float32), _c(b, np.float32)
    assert a.shape == b.shape
    y = np.empty(x.shape, dtype=np.float64)
    _load().oracle_chain_f64(_p(x), _p(y), x.size, _p(a), _p(b), a.size, int(relu_even))
    return y


def chain_f32fma(x, a, b, relu_even: bool = True) -> np.ndarray:
    """Same chain in fp32, one correctly rounded fma per stage."""
    x, a, b = _c(x, np.float32), _c(a, np.float32), _c(b, np.float32)
    y = np.empty(x.shape, dtype=np.float32)
    _load().oracle_chain_f32fma(_p(x), _p(y), x.size, _p(a), _p(b), a.size, int(relu_even))
    return y


def chain_fat_sink_f64(x, a, b, relu_even: bool, temps: int, lanes: int, with_abs: bool = False):
    """Sink of the fat probe ("C-05" section 3, fat row) in fp64: 4*lanes values,
    sink[4*lane + c] = sum over the lane's vectors q = lane, lane+lanes, ... of
    sum_j t_j, t_j = t_{j-1}/2 + y_{floor(jK/T)}.  With ``with_abs`` also the
    same sums of |t_j| (the error scale of an fp32 evaluation)."""
    x, a, b = _c(x, np.float32), _c(a, np.float32), _c(b, np.float32)
    assert a.shape == b.shape and lanes >= 1 and temps >= 0
    sink = np.empty(4 * lanes, dtype=np.float64)
    absd = np.empty(4 * lanes, dtype=np.float64) if with_abs else None
    _load().oracle_chain_fat_sink_f64(_p(x), x.size, _p(a), _p(b), a.size, int(relu_even), int(temps),
                                      int(lanes), _p(sink), _p(absd) if with_abs else None)
    return (sink, absd) if with_abs else sink


def chain_fat_sink_f32(x, a, b, relu_even: bool, temps: int, lanes: int) -> np.ndarray:
    """The same sink with every step one fp32 rounding, in the probe's order."""
    x, a, b = _c(x, np.float32), _c(a, np.float32), _c(b, np.float32)
    assert a.shape == b.shape and lanes >= 1 and temps >= 0
    sink = np.empty(4 * lanes, dtype=np.float32)
    _load().oracle_chain_fat_sink_f32(_p(x), x.size, _p(a), _p(b), a.size, int(relu_even), int(temps),
                                      int(lanes), _p(sink))
    return sink


# ---------------------------------------------------------------- gemm + epilogue

def gelu(z: float) -> float:
    return _load().oracle_gelu(float(z))


def half_to_double(h: int) -> float:
    return _load().oracle_half_to_double(int(h))


def bf16_to_double(h: int) -> float:
    return _load().oracle_bf16_to_double(int(h))


def gemm_f64(A, B) -> np.ndarray:
    """C = A.B in fp64 from fp16 bit arrays A [M,K], B [K,N]."""
    A, B = _c(A, np.uint16), _c(B, np.uint16)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    C = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm_f64(_p(A), _p(B), M, N, K, _p(C))
    return C


def gemm_epilogue_f64(A, B, bias, R) -> np.ndarray:
    """Y = GELU(A.B + bias) + R in fp64 from fp16 bit arrays."""
    A, B, bias, R = (_c(t, np.uint16) for t in (A, B, bias, R))
    M, K = A.shape
    N = B.shape[1]
    assert B.shape[0] == K and bias.shape == (N,) and R.shape == (M, N)
    Y = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm_epilogue_f64(_p(A), _p(B), _p(bias), _p(R), M, N, K, _p(Y))
    return Y


def gemm_epilogue_f64_matmul(A, B, bias, R) -> np.ndarray:
    """The same Y with the product step taken by numpy's fp64 matrix product
    (a library primitive; fp16 -> fp64 is exact) and the bias, GELU and
    residual stages by the C oracle: fast enough for 4096^3 in a test."""
    A, B, bias, R = (_c(t, np.uint16) for t in (A, B, bias, R))
    M, K = A.shape
    N = B.shape[1]
    assert B.shape[0] == K and bias.shape == (N,) and R.shape == (M, N)
    C = np.ascontiguousarray(np.matmul(A.view(np.float16).astype(np.float64),
                                       B.view(np.float16).astype(np.float64)))
    Y = np.empty((M, N), dtype=np.float64)
    _load().oracle_epilogue_on_product_f64(_p(C), _p(bias), _p(R), M, N, _p(Y))
    return Y


def gemm_epilogue_at(A, B, bias, R, rows, cols) -> np.ndarray:
    """Y at sampled (rows[t], cols[t]) positions."""
    A, B, bias, R = (_c(t, np.uint16) for t in (A, B, bias, R))
    M, K = A.shape
    N = B.shape[1]
    rows, cols = _c(rows, np.int64), _c(cols, np.int64)
    assert rows.shape == cols.shape
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < M and cols.min() >= 0 and cols.max() < N)
    out = np.empty(rows.shape, dtype=np.float64)
    _load().oracle_gemm_epilogue_at(_p(A), _p(B), _p(bias), _p(R), M, N, K,
                                    _p(rows), _p(cols), rows.size, _p(out))
    return out


# ---------------------------------------------------------------- causal softmax

def causal_softmax_f64(scores, scale: float) -> np.ndarray:
    """out [BH,S,S] fp64 from bf16 bits scores [BH,S,S]."""
    s = _c(scores, np.uint16)
    BH, S, S2 = s.shape
    assert S == S2
    out = np.empty(s.shape, dtype=np.float64)
    _load().oracle_causal_softmax_f64(_p(s), BH, S, float(scale), _p(out))
    return out


def causal_softmax_rows(scores, scale: float, row_ids) -> np.ndarray:
    """Rows r = bh*S + i of the causal softmax, shape [len(row_ids), S]."""
    s = _c(scores, np.uint16)
    BH, S, _ = s.shape
    rid = _c(row_ids, np.int64)
    assert rid.size == 0 or (rid.min() >= 0 and rid.max() < BH * S)
    out = np.empty((rid.size, S), dtype=np.float64)
    _load().oracle_causal_softmax_rows(_p(s), S, float(scale), _p(rid), rid.size, _p(out))
    return out


def causal_mask01(S: int) -> np.ndarray:
    """The causal mask of one [S,S] head: 1 where key j <= query i, else 0."""
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    return (j <= i).astype(np.float64)


# ---------------------------------------------------------------- causal attention

def causal_attention_rows(Q, K, V, scale: float, row_ids) -> np.ndarray:
    """Rows r = bh*S + i of O = softmax(scale * Q K^T, causal) V in fp64, from
    bf16 bits Q, K, V [BH, S, D]; shape [len(row_ids), D]."""
    q, k, v = _c(Q, np.uint16), _c(K, np.uint16), _c(V, np.uint16)
    assert q.shape == k.shape == v.shape and q.ndim == 3
    BH, S, D = q.shape
    rid = _c(row_ids, np.int64)
    assert rid.size == 0 or (rid.min() >= 0 and rid.max() < BH * S)
    out = np.empty((rid.size, D), dtype=np.float64)
    rc = _load().oracle_causal_attention_rows(_p(q), _p(k), _p(v), S, D, float(scale), _p(rid),
                                              rid.size, _p(out))
    if rc != 0:
        raise MemoryError("oracle_causal_attention_rows: allocation failed")
    return out


def causal_attention_f64(Q, K, V, scale: float) -> np.ndarray:
    """All rows of O, shape [BH, S, D] (small inputs only)."""
    BH, S, D = np.shape(Q)
    return causal_attention_rows(Q, K, V, scale, np.arange(BH * S)).reshape(BH, S, D)


# ---------------------------------------------------------------- RMSNorm

def rmsnorm_f64(x, g, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * g per row, fp64, from fp32 x [rows, d] and g [d]."""
    x, g = _c(x, np.float32), _c(g, np.float32)
    rows, d = x.shape
    assert g.shape == (d,)
    y = np.empty((rows, d), dtype=np.float64)
    _load().oracle_rmsnorm_f64(_p(x), _p(g), rows, d, float(eps), _p(y))
    return y
