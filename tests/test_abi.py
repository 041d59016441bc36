"""The C-ABI library without a GPU: it loads, exports every symbol the header declares, and
rejects bad arguments with the documented status before launching anything."""

import ctypes
import os
import re

import pytest

from mla_decode_decoupled_amd import _lib
from mla_decode_decoupled_amd._lib import (MLA_BF16, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE,
                                           MLA_F32, MLA_OK, MlaConfig, lib)

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    return set(re.findall(r"^\s*(?:const char\*|mla_status|size_t|int32_t)\s+(mla_\w+)\s*\(", text, re.M))


def test_header_symbols_exported():
    names = _declared()
    assert {"mla_rope_append", "mla_absorb_q", "mla_decode_attn", "mla_out_proj",
            "mla_decode_attn_workspace_size", "mla_status_string", "mla_last_error", "mla_version"} <= names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_config_struct_layout():
    assert ctypes.sizeof(MlaConfig) == 40
    assert MlaConfig.rope_base.offset == 24 and MlaConfig.softmax_scale.offset == 32


def cfg(**kw):
    base = dict(n_heads=128, d_nope=128, d_latent=512, d_rope=64, d_v=128, dtype=MLA_BF16, rope_base=10000.0,
                softmax_scale=0.0721687836, reserved=0)
    base.update(kw)
    return MlaConfig(**base)


@pytest.mark.parametrize("bad,code", [
    (dict(n_heads=0), MLA_ERR_INVALID_ARG),
    (dict(d_latent=-1), MLA_ERR_INVALID_ARG),
    (dict(d_rope=7), MLA_ERR_INVALID_ARG),
    (dict(dtype=9), MLA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), MLA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), MLA_ERR_INVALID_ARG),
    (dict(rope_base=-1.0), MLA_ERR_INVALID_ARG),
    (dict(reserved=1), MLA_ERR_INVALID_ARG),
    (dict(d_latent=2048), MLA_ERR_UNSUPPORTED),
    (dict(d_nope=512), MLA_ERR_UNSUPPORTED),
])
def test_bad_config_rejected_by_every_call(bad, code):
    c = cfg(**bad)
    assert lib.mla_rope_append(c, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
    assert lib.mla_absorb_q(c, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
    assert lib.mla_decode_attn(c, 1, 1, FAKE, FAKE, FAKE, FAKE, 10, 0, None, 0, FAKE, None, None) == code
    assert lib.mla_out_proj(c, 1, FAKE, FAKE, FAKE, 0, None, None, None) == code
    assert lib.mla_decode_attn_workspace_size(c, 1, 1, 10, 0) == 0
    assert lib.mla_last_error() != b""


def test_null_config():
    assert lib.mla_absorb_q(None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MLA_ERR_INVALID_ARG
    assert b"NULL" in lib.mla_last_error()


def test_null_pointers_and_negative_sizes():
    c = cfg()
    assert lib.mla_rope_append(c, 1, 1, None, FAKE, FAKE, FAKE, FAKE, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_rope_append(c, -1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(c, 2, FAKE, FAKE, None, FAKE, FAKE, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(c, -2, FAKE, FAKE, FAKE, FAKE, FAKE, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_decode_attn(c, 1, 1, FAKE, None, FAKE, FAKE, 10, 0, None, 0, FAKE, None, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_decode_attn(c, 1, 1, FAKE, FAKE, FAKE, FAKE, 10, 0, None, 0, None, None, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_out_proj(c, 1, None, FAKE, FAKE, 0, None, None, None) == MLA_ERR_INVALID_ARG


def test_decode_attn_shape_rules():
    c = cfg()
    # max_seq_len below n_q
    assert lib.mla_decode_attn(c, 1, 8, FAKE, FAKE, FAKE, FAKE, 4, 0, None, 0, FAKE, None, None) == MLA_ERR_INVALID_ARG
    # split count outside [0, 256]
    assert lib.mla_decode_attn(c, 1, 1, FAKE, FAKE, FAKE, FAKE, 4096, 999, None, 0, FAKE, None, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_decode_attn(c, 1, 1, FAKE, FAKE, FAKE, FAKE, 4096, -1, None, 0, FAKE, None, None) == MLA_ERR_INVALID_ARG


def test_workspace_rules():
    c = cfg()
    need = lib.mla_decode_attn_workspace_size(c, 4, 1, 131073, 64)
    assert need > 0
    assert need == lib.mla_decode_attn_workspace_size(c, 4, 1, 131073, 64)
    assert lib.mla_decode_attn(c, 4, 1, FAKE, FAKE, FAKE, FAKE, 131073, 64, None, need, FAKE, None, None) == MLA_ERR_WORKSPACE
    assert lib.mla_decode_attn(c, 4, 1, FAKE, FAKE, FAKE, FAKE, 131073, 64, FAKE, need - 1, FAKE, None, None) == MLA_ERR_WORKSPACE
    # a single split needs no workspace
    assert lib.mla_decode_attn_workspace_size(c, 1, 1, 100, 1) == 0


def test_w_o_projection_arguments_must_agree():
    """d_model > 0 needs both w_o and u, d_model = 0 neither; checked before any launch."""
    c = cfg()
    for d_model, w_o, u in ((7168, None, FAKE), (7168, FAKE, None), (0, FAKE, None), (0, None, FAKE),
                            (0, FAKE, FAKE), (-1, None, None), (-5, FAKE, FAKE)):
        assert lib.mla_out_proj(c, 1, FAKE, FAKE, FAKE, d_model, w_o, u, None) == MLA_ERR_INVALID_ARG, (d_model, w_o, u)
        assert b"W_O" in lib.mla_last_error() or b"d_model" in lib.mla_last_error()


def test_empty_work_returns_ok_without_launch():
    c = cfg(dtype=MLA_F32)
    assert lib.mla_rope_append(c, 0, 5, None, None, None, None, None, None) == MLA_OK
    assert lib.mla_absorb_q(c, 0, None, None, None, None, None, None) == MLA_OK
    assert lib.mla_decode_attn(c, 0, 1, None, None, None, None, 0, 0, None, 0, None, None, None) == MLA_OK
    assert lib.mla_out_proj(c, 0, None, None, None, 0, None, None, None) == MLA_OK
    assert lib.mla_last_error() == b""


def test_status_strings():
    for s in range(5):
        assert lib.mla_status_string(s).startswith(b"MLA_")
    assert b"gfx950" in lib.mla_version()


def test_python_wrappers_validate_before_calling():
    torch = pytest.importorskip("torch")
    import mla_decode_decoupled_amd as mla
    c = mla.make_config(4, 16, 32, 8, 16, "f32")
    with pytest.raises(ValueError):
        mla.mla_absorb_q(c, torch.zeros(1, 4, 16), torch.zeros(1, 4, 8), torch.zeros(1, dtype=torch.int32),
                         torch.zeros(4, 16, 32), torch.zeros(1, 4, 40))   # host tensors are refused


def test_projection_and_advance_arguments():
    """The upstream-projection calls and the decode advance validate before launching."""
    c = cfg()
    ws = lib.mla_project_workspace_size(c, 4, 7168, 1536)
    assert ws >= 4 * 576 * 4 and ws >= 4 * 1536 * 2 and ws % 256 == 0
    assert lib.mla_project_workspace_size(cfg(n_heads=0), 4, 7168, 0) == 0
    assert lib.mla_project_workspace_size(c, 4, 0, 0) == 0
    # bad config, NULL pointers, negative sizes, missing or short workspace
    assert lib.mla_project_kv_append(cfg(d_rope=7), 1, 1, 7168, FAKE, FAKE, FAKE, None, 1e-6, FAKE, FAKE, FAKE,
                                     FAKE, ws, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_project_kv_append(c, 1, 1, 7168, None, FAKE, FAKE, None, 1e-6, FAKE, FAKE, FAKE, FAKE, ws,
                                     None) == MLA_ERR_INVALID_ARG
    assert lib.mla_project_kv_append(c, 1, 1, 7168, FAKE, FAKE, None, None, 1e-6, FAKE, FAKE, FAKE, FAKE, ws,
                                     None) == MLA_ERR_INVALID_ARG   # W_KR needed when d_rope > 0
    assert lib.mla_project_kv_append(c, -1, 1, 7168, FAKE, FAKE, FAKE, None, 1e-6, FAKE, FAKE, FAKE, FAKE, ws,
                                     None) == MLA_ERR_INVALID_ARG
    assert lib.mla_project_kv_append(c, 1, 1, 7168, FAKE, FAKE, FAKE, FAKE, -1.0, FAKE, FAKE, FAKE, FAKE, ws,
                                     None) == MLA_ERR_INVALID_ARG   # negative eps with a norm
    assert lib.mla_project_kv_append(c, 4, 1, 7168, FAKE, FAKE, FAKE, None, 1e-6, FAKE, FAKE, FAKE, None, ws,
                                     None) == MLA_ERR_WORKSPACE
    assert lib.mla_project_kv_append(c, 4, 1, 7168, FAKE, FAKE, FAKE, None, 1e-6, FAKE, FAKE, FAKE, FAKE,
                                     4 * 576 * 4 - 1, None) == MLA_ERR_WORKSPACE
    assert lib.mla_project_q(cfg(softmax_scale=0.0), 1, 7168, 0, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, 0,
                             None) == MLA_ERR_INVALID_ARG
    assert lib.mla_project_q(c, 1, 7168, 1536, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                             None) == MLA_ERR_INVALID_ARG   # d_q > 0 without W_DQ
    assert lib.mla_project_q(c, 1, 7168, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                             None) == MLA_ERR_INVALID_ARG   # W_DQ with d_q = 0
    assert lib.mla_project_q(c, 1, 7168, 1536, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws,
                             None) == MLA_ERR_INVALID_ARG
    assert lib.mla_project_q(c, 4, 7168, 1536, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4 * 1536 * 2 - 1,
                             None) == MLA_ERR_WORKSPACE
    assert lib.mla_project_q(c, -1, 7168, 0, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_decode_advance(-1, 1, FAKE, FAKE, 0, None, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_decode_advance(1, -1, FAKE, FAKE, 0, None, None) == MLA_ERR_INVALID_ARG
    # empty work is a no-op
    assert lib.mla_project_kv_append(c, 0, 3, 7168, None, None, None, None, 1e-6, None, None, None, None, 0,
                                     None) == MLA_OK
    assert lib.mla_project_q(c, 0, 7168, 0, None, None, None, None, None, None, None, 0, None) == MLA_OK
    assert lib.mla_decode_advance(4, 0, FAKE, FAKE, 4, FAKE, None) == MLA_OK
    assert lib.mla_decode_advance(4, 1, None, None, 4, None, None) == MLA_OK
    assert lib.mla_last_error() == b""


def test_explicit_prefill_arguments():
    c = cfg()
    ws = lib.mla_prefill_explicit_workspace_size(c, 2, 2048, 4096)
    assert ws == 2 * 2 * 4096 * 128 * 128 * 2
    assert lib.mla_prefill_explicit_workspace_size(cfg(dtype=MLA_F32), 2, 2048, 4096) == 0   # not covered
    assert lib.mla_prefill_explicit_workspace_size(c, 2, 2048, 100) == 0                     # max_seq_len < n_q
    args = lambda c, ws_ptr, ws_bytes, o=FAKE, d_model=0, w_o=None, u=None: (  # noqa: E731
        c, 2, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, ws_ptr, ws_bytes, o, None, d_model, w_o, u, None)
    assert lib.mla_prefill_explicit(*args(cfg(dtype=MLA_F32), FAKE, ws)) == MLA_ERR_UNSUPPORTED
    assert lib.mla_prefill_explicit(*args(cfg(d_rope=32), FAKE, ws)) == MLA_ERR_UNSUPPORTED
    assert lib.mla_prefill_explicit(*args(c, None, ws)) == MLA_ERR_WORKSPACE
    assert lib.mla_prefill_explicit(*args(c, FAKE, ws - 1)) == MLA_ERR_WORKSPACE
    assert lib.mla_prefill_explicit(*args(c, FAKE, ws, o=None)) == MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_explicit(c, 2, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE, FAKE, ws, FAKE, None,
                                    0, None, None, None) == MLA_ERR_INVALID_ARG                   # max_seq_len < n_q
    # the optional W_O output: all three or none
    assert lib.mla_prefill_explicit(*args(c, FAKE, ws, d_model=7168)) == MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_explicit(*args(c, FAKE, ws, w_o=FAKE, u=FAKE)) == MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_explicit(*args(c, FAKE, ws, d_model=-1)) == MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_explicit(*args(c, FAKE, ws, d_model=7168, w_o=FAKE, u=ctypes.c_void_p(0x1004))) \
        == MLA_ERR_INVALID_ARG                                                                    # misaligned u
    # 2 H column tiles in the rebuild grid's second dimension
    assert lib.mla_prefill_explicit(*args(cfg(n_heads=40000), FAKE, ws)) == MLA_ERR_UNSUPPORTED
    assert b"32767" in lib.mla_last_error()
    odd = ctypes.c_void_p(0x1008)
    assert lib.mla_prefill_explicit(c, 2, 2048, odd, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, ws, FAKE, None,
                                    0, None, None, None) == MLA_ERR_INVALID_ARG                   # misaligned
    assert lib.mla_prefill_explicit(c, 0, 2048, None, None, None, None, None, 0, None, None, None, 0, None, None,
                                    0, None, None, None) == MLA_OK


def test_prefill_route():
    """The explicit form is preferred from the measured row count on, only where it is compiled."""
    c = cfg()
    assert lib.mla_prefill_prefers_explicit(c, 2, 2048, 4096) == 1
    assert lib.mla_prefill_prefers_explicit(c, 64, 1, 8192) == 0            # decode: absorbed
    assert lib.mla_prefill_prefers_explicit(c, 2, 16, 4096) == 0
    assert lib.mla_prefill_prefers_explicit(cfg(dtype=MLA_F32), 2, 2048, 4096) == 0
    assert lib.mla_prefill_prefers_explicit(cfg(d_rope=32), 2, 2048, 4096) == 0
    assert lib.mla_prefill_prefers_explicit(c, 2, 2048, 100) == 0           # max_seq_len < n_q
    assert lib.mla_prefill_prefers_explicit(None, 2, 2048, 4096) == 0
    switch = next(n for n in range(1, 4097) if lib.mla_prefill_prefers_explicit(c, 1, n, 4096))
    assert all(lib.mla_prefill_prefers_explicit(c, 1, n, 4096) for n in (switch, switch + 1, 4096))


def test_decode_step_arguments():
    """mla_decode_step validates like the four calls it stands for, before any launch."""
    c = cfg()
    need = lib.mla_decode_step_workspace_size(c, 1, 1, 4097, 0)
    attn = lib.mla_decode_attn_workspace_size(c, 1, 1, 4097, 0)
    assert need >= attn + 8 and need == lib.mla_decode_step_workspace_size(c, 1, 1, 4097, 0)
    assert lib.mla_decode_step_workspace_size(c, 1, 8, 4, 0) == 0          # max_seq_len < n_q
    assert lib.mla_decode_step_workspace_size(cfg(reserved=1), 1, 1, 10, 0) == 0
    # a single chunk still needs the position scratch
    assert lib.mla_decode_step_workspace_size(c, 2, 1, 100, 1) >= 16

    def call(c, ws_ptr, ws_bytes, batch=1, n_q=1, max_len=4097, n_splits=0, c_new=FAKE, o=FAKE, z=FAKE):
        return lib.mla_decode_step(c, batch, n_q, c_new, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, max_len,
                                   n_splits, ws_ptr, ws_bytes, FAKE, z, None, o, None)

    assert call(cfg(reserved=1), FAKE, need) == MLA_ERR_INVALID_ARG
    assert call(c, None, need) == MLA_ERR_WORKSPACE
    assert call(c, FAKE, need - 1) == MLA_ERR_WORKSPACE
    assert call(c, FAKE, need, c_new=None) == MLA_ERR_INVALID_ARG
    assert call(c, FAKE, need, o=None) == MLA_ERR_INVALID_ARG
    assert call(c, FAKE, need, z=None) == MLA_ERR_INVALID_ARG
    assert call(c, FAKE, need, n_q=8, max_len=4) == MLA_ERR_INVALID_ARG
    assert call(c, FAKE, need, n_splits=999) == MLA_ERR_INVALID_ARG
    assert call(c, FAKE, need, batch=-1) == MLA_ERR_INVALID_ARG
    assert call(c, FAKE, need, batch=300, n_q=300) == MLA_ERR_UNSUPPORTED
    assert lib.mla_decode_step(c, 0, 1, None, None, None, None, None, None, None, None, None, 0, 0, None, 0, None,
                               None, None, None, None) == MLA_OK


def test_project_inputs_arguments():
    """mla_project_inputs validates like mla_project_kv_append and mla_project_q together."""
    c = cfg()
    need = lib.mla_project_inputs_workspace_size(c, 4, 7168, 1536)
    assert need >= 4 * 576 * 4 + 4 * 1536 * 2
    assert lib.mla_project_inputs_workspace_size(c, 0, 7168, 1536) == 0

    def call(ws_bytes=need, d_q=1536, w_dq=FAKE, h=FAKE, q_nope=FAKE, eps=1e-6, norm=None, batch=2, n_new=2):
        return lib.mla_project_inputs(c, batch, n_new, 7168, d_q, h, FAKE, FAKE, norm, eps, FAKE, FAKE, FAKE, w_dq,
                                      FAKE, FAKE, q_nope, FAKE, FAKE, ws_bytes, None)

    assert call(d_q=1536, w_dq=None) == MLA_ERR_INVALID_ARG      # w_dq exactly when d_q > 0
    assert call(d_q=0, w_dq=FAKE) == MLA_ERR_INVALID_ARG
    assert call(h=None) == MLA_ERR_INVALID_ARG
    assert call(q_nope=None) == MLA_ERR_INVALID_ARG
    assert call(norm=FAKE, eps=float("nan")) == MLA_ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == MLA_ERR_WORKSPACE
    assert call(batch=-1) == MLA_ERR_INVALID_ARG
    assert call(batch=0) == MLA_OK


CEIL_HEADER = os.path.join(os.path.dirname(HEADER), "mla_ceilings.h")


def test_ceilings_library_exports_and_validation():
    """The ceiling microbenchmark library exports what its header declares and rejects bad
    arguments before launching."""
    from mla_decode_decoupled_amd import _ceilings as C
    names = set(re.findall(r"^\s*int\s+(mla_\w+)\s*\(", open(CEIL_HEADER).read(), re.M))
    assert names == {"mla_ceiling_mfma", "mla_ceiling_stream", "mla_ceiling_lds"}
    for n in names:
        assert hasattr(C.lib, n) and n in C.SIGNATURES
    assert C.lib.mla_ceiling_mfma(1, 4, 0, 10, FAKE, FAKE, FAKE, None) == 1        # no workgroups
    assert C.lib.mla_ceiling_mfma(1, 4, 256, 10, None, FAKE, FAKE, None) == 1
    assert C.lib.mla_ceiling_mfma(3, 4, 256, 10, FAKE, FAKE, FAKE, None) == 2      # 3 waves per SIMD
    assert C.lib.mla_ceiling_mfma(2, 1, 256, 10, FAKE, FAKE, FAKE, None) == 2
    assert C.lib.mla_ceiling_stream(0, 8, 256, FAKE, 100, FAKE, None, None) == 1   # not a multiple of 16
    assert C.lib.mla_ceiling_stream(0, 5, 256, FAKE, 1024, FAKE, None, None) == 2
    assert C.lib.mla_ceiling_stream(1, 2, 256, FAKE, 36864, FAKE, None, None) == 1  # stamps needed
    assert C.lib.mla_ceiling_stream(1, 2, 256, FAKE, 1000, FAKE, FAKE, None) == 1   # not whole tiles
    assert C.lib.mla_ceiling_stream(1, 4, 256, FAKE, 36864, FAKE, FAKE, None) == 2
    assert C.lib.mla_ceiling_stream(7, 2, 256, FAKE, 36864, FAKE, FAKE, None) == 2
    assert C.lib.mla_ceiling_lds(0, 0, 10, FAKE, FAKE, None) == 1
    assert C.lib.mla_ceiling_lds(0, 256, 10, None, FAKE, None) == 1
    assert C.lib.mla_ceiling_lds(2, 256, 10, FAKE, FAKE, None) == 2


def test_decode_step_noalloc_arguments():
    """The no-allocation step validates like mla_decode_step and rejects, before touching the GPU,
    a plan whose workspace exceeds the library's scratch."""
    c = cfg()
    assert _lib.MLA_NOALLOC_SCRATCH_BYTES == 64 << 20

    def call(c, batch=1, n_q=1, max_len=4097, n_splits=0, c_new=FAKE, o=FAKE):
        return lib.mla_decode_step_noalloc(c, batch, n_q, c_new, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           max_len, n_splits, FAKE, FAKE, None, o, None)

    assert call(cfg(reserved=1)) == MLA_ERR_INVALID_ARG
    assert call(c, c_new=None) == MLA_ERR_INVALID_ARG
    assert call(c, o=None) == MLA_ERR_INVALID_ARG
    assert call(c, n_q=8, max_len=4) == MLA_ERR_INVALID_ARG
    assert call(c, n_splits=999) == MLA_ERR_INVALID_ARG
    assert call(c, batch=0) == MLA_OK
    # 16 rows x 256 chunks of fp32 partials: far more than the scratch holds
    need = lib.mla_decode_step_workspace_size(c, 16, 1, 65536, 256)
    assert need > _lib.MLA_NOALLOC_SCRATCH_BYTES
    assert call(c, batch=16, max_len=65536, n_splits=256) == MLA_ERR_UNSUPPORTED
    assert b"scratch" in lib.mla_last_error()


STAMPS_HEADER = os.path.join(os.path.dirname(HEADER), "mla_stamps.h")


def test_stamps_library_exports_and_validation():
    """The phase-stamp build exports every call of mla.h and of mla_stamps.h, reports the size of its
    stamp array, and rejects a null or short destination before touching the device."""
    import ctypes

    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "mla_decode_decoupled_amd",
                        "libmla_stamps.so")
    lib = ctypes.CDLL(path)
    names = set(re.findall(r"^\s*(?:int|size_t)\s+(mla_\w+)\s*\(", open(STAMPS_HEADER).read(), re.M))
    assert names == {"mla_phase_stamps_bytes", "mla_phase_stamps_clear", "mla_phase_stamps_read"}
    main = set(re.findall(r"^\s*(?:mla_status|size_t|int|const char\s*\*)\s+(mla_\w+)\s*\(", open(HEADER).read(), re.M))
    assert main
    for n in names | main:
        assert hasattr(lib, n), n
    lib.mla_phase_stamps_bytes.restype = ctypes.c_size_t
    lib.mla_phase_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    n = lib.mla_phase_stamps_bytes()
    assert n == 8192 * 16 * 8
    assert lib.mla_phase_stamps_read(None, n) == MLA_ERR_INVALID_ARG
    buf = ctypes.create_string_buffer(16)
    assert lib.mla_phase_stamps_read(buf, 16) == MLA_ERR_INVALID_ARG
