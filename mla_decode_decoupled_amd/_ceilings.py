"""ctypes binding of libmla_ceilings.so (include/mla_ceilings.h): the MFMA-issue and HBM-streaming
microbenchmarks. Argument marshalling only; raises on import when the library is not built."""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmla_ceilings.so")

_VP = ctypes.c_void_p
_I = ctypes.c_int

SIGNATURES = {
    "mla_ceiling_mfma": (ctypes.c_int, [_I, _I, _I, _I, _VP, _VP, _VP, _VP]),
    "mla_ceiling_stream": (ctypes.c_int, [_I, _I, _I, _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "mla_ceiling_lds": (ctypes.c_int, [_I, _I, _I, _VP, _VP, _VP]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmla_ceilings.so not found at {LIB_PATH}; build it with "
                          "`python mla_decode_decoupled_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{where} returned {rc}")


def mfma(waves_per_simd: int, n_acc: int, n_workgroups: int, iters: int, operands, stamps, sink, stream) -> None:
    """Enqueue the MFMA issue kernel; tensors are device tensors sized as the header states."""
    _check(lib.mla_ceiling_mfma(waves_per_simd, n_acc, n_workgroups, iters, operands.data_ptr(),
                                stamps.data_ptr(), sink.data_ptr(), stream), "mla_ceiling_mfma")


def stream(mode: int, depth: int, n_workgroups: int, src, bytes_per_workgroup: int, sink, stamps, stream_) -> None:
    """Enqueue one streaming-read kernel (mode 0: vector loads, 1: the LDS tile ring)."""
    _check(lib.mla_ceiling_stream(mode, depth, n_workgroups, src.data_ptr(), bytes_per_workgroup, sink.data_ptr(),
                                  None if stamps is None else stamps.data_ptr(), stream_), "mla_ceiling_stream")


def lds(mode: int, n_workgroups: int, iters: int, sink, stamps, stream_) -> None:
    """Enqueue the LDS read-throughput kernel (mode 0: ds_read_b128, 1: ds_read_b64_tr_b16)."""
    _check(lib.mla_ceiling_lds(mode, n_workgroups, iters, sink.data_ptr(), stamps.data_ptr(), stream_),
           "mla_ceiling_lds")
