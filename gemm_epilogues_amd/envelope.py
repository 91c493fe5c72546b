"""Binding of libfcenv.so (C ABI in include/fc_envelope.h): reference rates.

Stream probes (copy, pure write, mixed read/write, pure read) and an MFMA
probe on random operands.  They carry none of the method's arithmetic; the
benchmark times them beside the hot-path kernels to state what fraction of the
reachable bandwidth or matrix rate each kernel attains.  Argument marshalling
only, like the main binding.
"""
from __future__ import annotations

import ctypes
import os

import gemm_epilogues_amd as fc   # loads torch first, so both libraries share its HIP runtime

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfcenv.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python gemm_epilogues_amd/build.py` first")
_lib = ctypes.CDLL(LIB_PATH)

_P, _SZ, _I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_lib.fce_chunk_bytes.restype, _lib.fce_chunk_bytes.argtypes = _SZ, []
_lib.fce_mix.restype, _lib.fce_mix.argtypes = _I, [_P, _SZ, _P, _SZ, _P]
_lib.fce_read.restype, _lib.fce_read.argtypes = _I, [_P, _SZ, _P, _P]
_lib.fce_flat.restype, _lib.fce_flat.argtypes = _I, [_P, _P, _SZ, _P]
_lib.fce_mfma.restype, _lib.fce_mfma.argtypes = _I, [_P, _I, _P]
_lib.fce_mfma_sink_floats.restype, _lib.fce_mfma_sink_floats.argtypes = _SZ, []
_lib.fce_mfma_flops.restype, _lib.fce_mfma_flops.argtypes = ctypes.c_double, [_I]
_lib.fce_empty.restype, _lib.fce_empty.argtypes = _I, [_I, _P, _P]
_lib.fce_empty_n.restype, _lib.fce_empty_n.argtypes = _I, [_I, _I, _P, _P]
_lib.fce_mix_n.restype, _lib.fce_mix_n.argtypes = _I, [_P, _SZ, _P, _SZ, _I, _P]

EXPORTED = ("fce_chunk_bytes", "fce_mix", "fce_read", "fce_flat", "fce_mfma", "fce_mfma_sink_floats",
            "fce_mfma_flops", "fce_empty", "fce_empty_n", "fce_mix_n")


def _addr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    return t.data_ptr()


def _stream(stream):
    return fc._stream(stream)


def fce_chunk_bytes() -> int:
    return int(_lib.fce_chunk_bytes())


def fce_mix(src, read_bytes: int, dst, write_bytes: int, stream=None) -> None:
    """Read `read_bytes` of src and write `write_bytes` of dst (whole chunks)."""
    fc._check(_lib.fce_mix(_addr(src), int(read_bytes), _addr(dst), int(write_bytes), _stream(stream)), "fce_mix")


def fce_read(src, read_bytes: int, sink, stream=None) -> None:
    fc._check(_lib.fce_read(_addr(src), int(read_bytes), _addr(sink), _stream(stream)), "fce_read")


def fce_flat(src, dst, nbytes: int, stream=None) -> None:
    """Flat stream of nbytes: a pure write of dst when src is None, else a copy."""
    fc._check(_lib.fce_flat(_addr(src) if src is not None else None, _addr(dst), int(nbytes), _stream(stream)),
              "fce_flat")


def fce_mfma_sink_floats() -> int:
    return int(_lib.fce_mfma_sink_floats())


def fce_mfma_flops(iters: int) -> float:
    return float(_lib.fce_mfma_flops(int(iters)))


def fce_mfma(sink, iters: int, stream=None) -> None:
    fc._check(_lib.fce_mfma(_addr(sink), int(iters), _stream(stream)), "fce_mfma")


def fce_empty(blocks: int, sink, stream=None) -> None:
    fc._check(_lib.fce_empty(int(blocks), _addr(sink), _stream(stream)), "fce_empty")


def fce_empty_n(blocks: int, n: int, sink, stream=None) -> None:
    """n empty kernels back to back from one call."""
    fc._check(_lib.fce_empty_n(int(blocks), int(n), _addr(sink), _stream(stream)), "fce_empty_n")


def fce_mix_n(src, read_bytes: int, dst, write_bytes: int, n: int, stream=None) -> None:
    """fce_mix n times back to back from one call."""
    fc._check(_lib.fce_mix_n(_addr(src), int(read_bytes), _addr(dst), int(write_bytes), int(n), _stream(stream)),
              "fce_mix_n")
