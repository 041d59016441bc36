"""ctypes binding of libmla.so (include/mla.h). Argument marshalling only.

Every compute step runs in the library's HIP kernels; torch provides device
memory and the current stream. If the library has not been built this module
raises on import, so a missing extension never falls back to anything else.
"""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# MLA_LIB_PATH selects another build of the same library (the host-sanitized libmla_asan.so, for the
# sanitizer run of the C-ABI checks); by default the in-tree libmla.so
LIB_PATH = os.environ.get("MLA_LIB_PATH") or os.path.join(PKG_DIR, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE = 3
MLA_ERR_HIP = 4

MLA_F32 = 0
MLA_BF16 = 1

MLA_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/mla.h


class MlaConfig(ctypes.Structure):
    _fields_ = [
        ("n_heads", ctypes.c_int32),
        ("d_nope", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("softmax_scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


assert ctypes.sizeof(MlaConfig) == 40

_VP = ctypes.c_void_p
_I32 = ctypes.c_int32

# name -> (restype, argtypes), mirroring include/mla.h
SIGNATURES = {
    "mla_version": (ctypes.c_char_p, []),
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_rope_append": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "mla_absorb_q": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "mla_decode_attn_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MlaConfig), _I32, _I32, _I32, _I32]),
    "mla_decode_attn": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _I32, _VP, _VP, _VP, _VP, _I32, _I32,
                                       _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "mla_out_proj": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _VP, _VP, _VP, _I32, _VP, _VP, _VP]),
    "mla_decode_step_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MlaConfig), _I32, _I32, _I32, _I32]),
    "mla_decode_step": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                       _VP, _VP, _I32, _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP, _VP, _VP]),
    "mla_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP,
                                               _VP, _VP, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP]),
    "mla_project_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MlaConfig), _I32, _I32, _I32]),
    "mla_project_kv_append": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _I32, _I32, _VP, _VP, _VP, _VP,
                                             ctypes.c_float, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "mla_project_q": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP,
                                     _VP, ctypes.c_size_t, _VP]),
    "mla_project_inputs_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MlaConfig), _I32, _I32, _I32]),
    "mla_project_inputs": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP,
                                          ctypes.c_float, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                          ctypes.c_size_t, _VP]),
    "mla_decode_advance": (ctypes.c_int, [_I32, _I32, _VP, _VP, _I32, _VP, _VP]),
    "mla_prefill_explicit_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MlaConfig), _I32, _I32, _I32]),
    "mla_prefill_explicit": (ctypes.c_int, [ctypes.POINTER(MlaConfig), _I32, _I32, _VP, _VP, _VP, _VP, _VP, _I32,
                                            _VP, _VP, _VP, ctypes.c_size_t, _VP, _VP, _I32, _VP, _VP, _VP]),
    "mla_prefill_prefers_explicit": (_I32, [ctypes.POINTER(MlaConfig), _I32, _I32, _I32]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmla.so not found at {LIB_PATH}; build it with `python -m mla_decode_decoupled_amd.build`"
        )
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.mla_status_string(status).decode()
        detail = lib.mla_last_error().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))


def check(status: int, where: str) -> None:
    if status != MLA_OK:
        raise MlaError(status, where)
