"""Torch-facing wrappers with the C-ABI's names (include/mla.h).

Each wrapper checks dtype, device, contiguity and shapes, raises ValueError on
a mismatch, and otherwise passes raw device pointers and the current HIP stream
to libmla. Nothing here computes any part of the attention.
"""

from __future__ import annotations

import math
from typing import Optional

import torch

from . import _lib
from ._lib import MLA_BF16, MLA_F32, MlaConfig, check, lib

_DT = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16}


def make_config(n_heads: int, d_nope: int, d_latent: int, d_rope: int, d_v: int, dtype: str = "bf16",
                rope_base: float = 10000.0, softmax_scale: Optional[float] = None) -> MlaConfig:
    """Layer description; softmax_scale defaults to 1/sqrt(d_nope + d_rope)."""
    code = {"f32": MLA_F32, "float32": MLA_F32, "bf16": MLA_BF16, "bfloat16": MLA_BF16}[dtype]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_nope + d_rope)
    return MlaConfig(n_heads, d_nope, d_latent, d_rope, d_v, code, float(rope_base), float(softmax_scale), 0)


def storage_dtype(cfg: MlaConfig) -> torch.dtype:
    return _DT[cfg.dtype]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def mla_rope_append(cfg: MlaConfig, c_new: torch.Tensor, k_rope_new: torch.Tensor, cache: torch.Tensor,
                    seq_off: torch.Tensor, len_before: torch.Tensor) -> None:
    """cache[seq_off[b] + len_before[b] + i] = [c_new[b, i] ; RoPE(k_rope_new[b, i])]."""
    dt = storage_dtype(cfg)
    if c_new.dim() != 3:
        raise ValueError("c_new must be [batch, n_new, d_latent]")
    B, n_new = c_new.shape[0], c_new.shape[1]
    dev = c_new.device
    _need(c_new, "c_new", dt, (B, n_new, cfg.d_latent))
    _need(k_rope_new, "k_rope_new", dt, (B, n_new, cfg.d_rope), dev)
    _need(cache, "cache", dt, None, dev)
    if cache.dim() != 2 or cache.shape[1] != cfg.d_latent + cfg.d_rope:
        raise ValueError("cache must be [rows, d_latent + d_rope]")
    _need(seq_off, "seq_off", torch.int64, (B,), dev)
    _need(len_before, "len_before", torch.int32, (B,), dev)
    check(lib.mla_rope_append(cfg, B, n_new, _ptr(c_new), _ptr(k_rope_new), _ptr(cache), _ptr(seq_off),
                              _ptr(len_before), _stream(cache)), "mla_rope_append")


def mla_absorb_q(cfg: MlaConfig, q_nope: torch.Tensor, q_rope: torch.Tensor, q_pos: torch.Tensor,
                 w_uk: torch.Tensor, q_packed: torch.Tensor) -> None:
    """q_packed[r, i] = [W_UK,i^T q_nope[r, i] ; RoPE_{q_pos[r]}(q_rope[r, i])]."""
    dt = storage_dtype(cfg)
    H = cfg.n_heads
    R = q_nope.shape[0] if q_nope.dim() == 3 else -1
    dev = q_nope.device
    _need(q_nope, "q_nope", dt, (R, H, cfg.d_nope))
    _need(q_rope, "q_rope", dt, (R, H, cfg.d_rope), dev)
    _need(q_pos, "q_pos", torch.int32, (R,), dev)
    _need(w_uk, "w_uk", dt, (H, cfg.d_nope, cfg.d_latent), dev)
    _need(q_packed, "q_packed", dt, (R, H, cfg.d_latent + cfg.d_rope), dev)
    check(lib.mla_absorb_q(cfg, R, _ptr(q_nope), _ptr(q_rope), _ptr(q_pos), _ptr(w_uk), _ptr(q_packed),
                           _stream(q_packed)), "mla_absorb_q")


def mla_decode_attn_workspace_size(cfg: MlaConfig, batch: int, n_q: int, max_seq_len: int, n_splits: int = 0) -> int:
    return int(lib.mla_decode_attn_workspace_size(cfg, batch, n_q, max_seq_len, n_splits))


def mla_decode_attn(cfg: MlaConfig, q_packed: torch.Tensor, cache: torch.Tensor, seq_off: torch.Tensor,
                    seq_len: torch.Tensor, max_seq_len: int, z: torch.Tensor, lse: Optional[torch.Tensor] = None,
                    n_splits: int = 0, workspace: Optional[torch.Tensor] = None) -> None:
    """Latent attention of q_packed [batch, n_q, H, d_latent + d_rope] over the cache; writes z (and lse)."""
    dt = storage_dtype(cfg)
    H, row = cfg.n_heads, cfg.d_latent + cfg.d_rope
    if q_packed.dim() != 4:
        raise ValueError("q_packed must be [batch, n_q, H, d_latent + d_rope]")
    B, n_q = q_packed.shape[0], q_packed.shape[1]
    dev = q_packed.device
    _need(q_packed, "q_packed", dt, (B, n_q, H, row))
    _need(cache, "cache", dt, None, dev)
    _need(seq_off, "seq_off", torch.int64, (B,), dev)
    _need(seq_len, "seq_len", torch.int32, (B,), dev)
    _need(z, "z", torch.float32, (B, n_q, H, cfg.d_latent), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, n_q, H), dev)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", workspace.dtype, None, dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    check(lib.mla_decode_attn(cfg, B, n_q, _ptr(q_packed), _ptr(cache), _ptr(seq_off), _ptr(seq_len),
                              int(max_seq_len), int(n_splits), _ptr(workspace), ws_bytes, _ptr(z), _ptr(lse),
                              _stream(z)), "mla_decode_attn")


def mla_out_proj(cfg: MlaConfig, z: torch.Tensor, w_uv: torch.Tensor, o: torch.Tensor,
                 w_o: Optional[torch.Tensor] = None, u: Optional[torch.Tensor] = None) -> None:
    """o[r, i] = W_UV,i z[r, i]; with w_o [d_model, H * d_v] and u [R, d_model] also
    u[r] = W_O concat_i(o[r, i])."""
    dt = storage_dtype(cfg)
    H = cfg.n_heads
    R = z.shape[0] if z.dim() == 3 else -1
    dev = z.device
    _need(z, "z", torch.float32, (R, H, cfg.d_latent))
    _need(w_uv, "w_uv", dt, (H, cfg.d_v, cfg.d_latent), dev)
    _need(o, "o", dt, (R, H, cfg.d_v), dev)
    if (w_o is None) != (u is None):
        raise ValueError("pass w_o and u together")
    d_model = 0
    if w_o is not None:
        if w_o.dim() != 2:
            raise ValueError("w_o must be [d_model, n_heads * d_v]")
        d_model = w_o.shape[0]
        _need(w_o, "w_o", dt, (d_model, H * cfg.d_v), dev)
        _need(u, "u", dt, (R, d_model), dev)
    check(lib.mla_out_proj(cfg, R, _ptr(z), _ptr(w_uv), _ptr(o), d_model, _ptr(w_o), _ptr(u), _stream(o)),
          "mla_out_proj")


def mla_decode_step_workspace_size(cfg: MlaConfig, batch: int, n_q: int, max_seq_len: int, n_splits: int = 0) -> int:
    return int(lib.mla_decode_step_workspace_size(cfg, batch, n_q, max_seq_len, n_splits))


def mla_decode_step(cfg: MlaConfig, c_new: torch.Tensor, k_rope_new: torch.Tensor, q_nope: torch.Tensor,
                    q_rope: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor, cache: torch.Tensor,
                    seq_off: torch.Tensor, seq_len: torch.Tensor, max_seq_len: int, q_packed: torch.Tensor,
                    z: torch.Tensor, o: torch.Tensor, lse: Optional[torch.Tensor] = None, n_splits: int = 0,
                    workspace: Optional[torch.Tensor] = None) -> None:
    """One decode step: append c_new / k_rope_new [batch, n_q, .] at positions seq_len - n_q + t,
    absorb q_nope / q_rope [batch * n_q, H, .], attend, project; writes q_packed, z, o (and lse)."""
    dt = storage_dtype(cfg)
    H, row = cfg.n_heads, cfg.d_latent + cfg.d_rope
    if c_new.dim() != 3:
        raise ValueError("c_new must be [batch, n_q, d_latent]")
    B, n_q = c_new.shape[0], c_new.shape[1]
    R = B * n_q
    dev = c_new.device
    _need(c_new, "c_new", dt, (B, n_q, cfg.d_latent))
    _need(k_rope_new, "k_rope_new", dt, (B, n_q, cfg.d_rope), dev)
    _need(q_nope, "q_nope", dt, (R, H, cfg.d_nope), dev)
    _need(q_rope, "q_rope", dt, (R, H, cfg.d_rope), dev)
    _need(w_uk, "w_uk", dt, (H, cfg.d_nope, cfg.d_latent), dev)
    _need(w_uv, "w_uv", dt, (H, cfg.d_v, cfg.d_latent), dev)
    _need(cache, "cache", dt, None, dev)
    if cache.dim() != 2 or cache.shape[1] != row:
        raise ValueError("cache must be [rows, d_latent + d_rope]")
    _need(seq_off, "seq_off", torch.int64, (B,), dev)
    _need(seq_len, "seq_len", torch.int32, (B,), dev)
    _need(q_packed, "q_packed", dt, (R, H, row), dev)
    _need(z, "z", torch.float32, (B, n_q, H, cfg.d_latent), dev)
    _need(o, "o", dt, (R, H, cfg.d_v), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, n_q, H), dev)
    wp, wb = _ws(workspace, dev)
    check(lib.mla_decode_step(cfg, B, n_q, _ptr(c_new), _ptr(k_rope_new), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                              _ptr(w_uv), _ptr(cache), _ptr(seq_off), _ptr(seq_len), int(max_seq_len), int(n_splits),
                              wp, wb, _ptr(q_packed), _ptr(z), _ptr(lse), _ptr(o), _stream(o)), "mla_decode_step")


def mla_decode_step_noalloc(cfg: MlaConfig, c_new: torch.Tensor, k_rope_new: torch.Tensor, q_nope: torch.Tensor,
                            q_rope: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor, cache: torch.Tensor,
                            seq_off: torch.Tensor, seq_len: torch.Tensor, max_seq_len: int, q_packed: torch.Tensor,
                            z: torch.Tensor, o: torch.Tensor, lse: Optional[torch.Tensor] = None,
                            n_splits: int = 0) -> None:
    """mla_decode_step without a workspace: the library's own per-device scratch array holds the
    split-K partials (calls that overlap on one GPU race; see include/mla.h)."""
    dt = storage_dtype(cfg)
    H, row = cfg.n_heads, cfg.d_latent + cfg.d_rope
    if c_new.dim() != 3:
        raise ValueError("c_new must be [batch, n_q, d_latent]")
    B, n_q = c_new.shape[0], c_new.shape[1]
    R = B * n_q
    dev = c_new.device
    _need(c_new, "c_new", dt, (B, n_q, cfg.d_latent))
    _need(k_rope_new, "k_rope_new", dt, (B, n_q, cfg.d_rope), dev)
    _need(q_nope, "q_nope", dt, (R, H, cfg.d_nope), dev)
    _need(q_rope, "q_rope", dt, (R, H, cfg.d_rope), dev)
    _need(w_uk, "w_uk", dt, (H, cfg.d_nope, cfg.d_latent), dev)
    _need(w_uv, "w_uv", dt, (H, cfg.d_v, cfg.d_latent), dev)
    _need(cache, "cache", dt, None, dev)
    if cache.dim() != 2 or cache.shape[1] != row:
        raise ValueError("cache must be [rows, d_latent + d_rope]")
    _need(seq_off, "seq_off", torch.int64, (B,), dev)
    _need(seq_len, "seq_len", torch.int32, (B,), dev)
    _need(q_packed, "q_packed", dt, (R, H, row), dev)
    _need(z, "z", torch.float32, (B, n_q, H, cfg.d_latent), dev)
    _need(o, "o", dt, (R, H, cfg.d_v), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, n_q, H), dev)
    if torch.cuda.current_device() != dev.index:
        raise ValueError(f"the tensors are on {dev}, but the current device is cuda:{torch.cuda.current_device()}")
    check(lib.mla_decode_step_noalloc(cfg, B, n_q, _ptr(c_new), _ptr(k_rope_new), _ptr(q_nope), _ptr(q_rope),
                                      _ptr(w_uk), _ptr(w_uv), _ptr(cache), _ptr(seq_off), _ptr(seq_len),
                                      int(max_seq_len), int(n_splits), _ptr(q_packed), _ptr(z), _ptr(lse), _ptr(o),
                                      _stream(o)), "mla_decode_step_noalloc")


def _ws(workspace: Optional[torch.Tensor], dev) -> tuple:
    if workspace is None:
        return None, 0
    _need(workspace, "workspace", workspace.dtype, None, dev)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def mla_project_workspace_size(cfg: MlaConfig, n_rows: int, d_model: int, d_q: int = 0) -> int:
    return int(lib.mla_project_workspace_size(cfg, n_rows, d_model, d_q))


def mla_project_kv_append(cfg: MlaConfig, h: torch.Tensor, w_dkv: torch.Tensor, w_kr: Optional[torch.Tensor],
                          cache: torch.Tensor, seq_off: torch.Tensor, len_before: torch.Tensor,
                          kv_norm_w: Optional[torch.Tensor] = None, kv_norm_eps: float = 1e-6,
                          workspace: Optional[torch.Tensor] = None) -> None:
    """cache[seq_off[b] + len_before[b] + i] = [RMSNorm(W_DKV h[b, i]) ; RoPE(W_KR h[b, i])]
    (no norm when kv_norm_w is None)."""
    dt = storage_dtype(cfg)
    if h.dim() != 3:
        raise ValueError("h must be [batch, n_new, d_model]")
    B, n_new, dm = h.shape
    dev = h.device
    _need(h, "h", dt)
    _need(w_dkv, "w_dkv", dt, (cfg.d_latent, dm), dev)
    if cfg.d_rope > 0 or w_kr is not None:
        _need(w_kr, "w_kr", dt, (cfg.d_rope, dm), dev)
    if kv_norm_w is not None:
        _need(kv_norm_w, "kv_norm_w", dt, (cfg.d_latent,), dev)
    _need(cache, "cache", dt, None, dev)
    if cache.dim() != 2 or cache.shape[1] != cfg.d_latent + cfg.d_rope:
        raise ValueError("cache must be [rows, d_latent + d_rope]")
    _need(seq_off, "seq_off", torch.int64, (B,), dev)
    _need(len_before, "len_before", torch.int32, (B,), dev)
    wp, wb = _ws(workspace, dev)
    check(lib.mla_project_kv_append(cfg, B, n_new, dm, _ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(kv_norm_w),
                                    float(kv_norm_eps), _ptr(cache), _ptr(seq_off), _ptr(len_before), wp, wb,
                                    _stream(cache)), "mla_project_kv_append")


def mla_project_q(cfg: MlaConfig, h: torch.Tensor, w_uq: torch.Tensor, w_qr: Optional[torch.Tensor],
                  q_nope: torch.Tensor, q_rope: Optional[torch.Tensor], w_dq: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> None:
    """q_nope / q_rope (unrotated) from h [R, d_model]: through c_Q = W_DQ h when w_dq is given,
    else straight from h."""
    dt = storage_dtype(cfg)
    H = cfg.n_heads
    if h.dim() != 2:
        raise ValueError("h must be [n_rows, d_model]")
    R, dm = h.shape
    dev = h.device
    _need(h, "h", dt)
    d_q = 0
    if w_dq is not None:
        if w_dq.dim() != 2:
            raise ValueError("w_dq must be [d_q, d_model]")
        d_q = w_dq.shape[0]
        _need(w_dq, "w_dq", dt, (d_q, dm), dev)
    K = d_q if d_q > 0 else dm
    _need(w_uq, "w_uq", dt, (H * cfg.d_nope, K), dev)
    _need(q_nope, "q_nope", dt, (R, H, cfg.d_nope), dev)
    if cfg.d_rope > 0 or w_qr is not None:
        _need(w_qr, "w_qr", dt, (H * cfg.d_rope, K), dev)
    if cfg.d_rope > 0 or q_rope is not None:
        _need(q_rope, "q_rope", dt, (R, H, cfg.d_rope), dev)
    wp, wb = _ws(workspace, dev)
    check(lib.mla_project_q(cfg, R, dm, d_q, _ptr(h), _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), _ptr(q_nope),
                            _ptr(q_rope), wp, wb, _stream(q_nope)), "mla_project_q")


def mla_project_inputs_workspace_size(cfg: MlaConfig, n_rows: int, d_model: int, d_q: int = 0) -> int:
    return int(lib.mla_project_inputs_workspace_size(cfg, n_rows, d_model, d_q))


def mla_project_inputs(cfg: MlaConfig, h: torch.Tensor, w_dkv: torch.Tensor, w_kr: Optional[torch.Tensor],
                       cache: torch.Tensor, seq_off: torch.Tensor, len_before: torch.Tensor, w_uq: torch.Tensor,
                       w_qr: Optional[torch.Tensor], q_nope: torch.Tensor, q_rope: Optional[torch.Tensor],
                       w_dq: Optional[torch.Tensor] = None, kv_norm_w: Optional[torch.Tensor] = None,
                       kv_norm_eps: float = 1e-6, workspace: Optional[torch.Tensor] = None) -> None:
    """mla_project_kv_append and mla_project_q on the same h [batch, n_new, d_model] in one call
    (the query rows are h viewed as [batch * n_new, d_model])."""
    dt = storage_dtype(cfg)
    H = cfg.n_heads
    if h.dim() != 3:
        raise ValueError("h must be [batch, n_new, d_model]")
    B, n_new, dm = h.shape
    R = B * n_new
    dev = h.device
    _need(h, "h", dt)
    _need(w_dkv, "w_dkv", dt, (cfg.d_latent, dm), dev)
    if cfg.d_rope > 0 or w_kr is not None:
        _need(w_kr, "w_kr", dt, (cfg.d_rope, dm), dev)
    if kv_norm_w is not None:
        _need(kv_norm_w, "kv_norm_w", dt, (cfg.d_latent,), dev)
    _need(cache, "cache", dt, None, dev)
    if cache.dim() != 2 or cache.shape[1] != cfg.d_latent + cfg.d_rope:
        raise ValueError("cache must be [rows, d_latent + d_rope]")
    _need(seq_off, "seq_off", torch.int64, (B,), dev)
    _need(len_before, "len_before", torch.int32, (B,), dev)
    d_q = 0
    if w_dq is not None:
        if w_dq.dim() != 2:
            raise ValueError("w_dq must be [d_q, d_model]")
        d_q = w_dq.shape[0]
        _need(w_dq, "w_dq", dt, (d_q, dm), dev)
    K = d_q if d_q > 0 else dm
    _need(w_uq, "w_uq", dt, (H * cfg.d_nope, K), dev)
    _need(q_nope, "q_nope", dt, (R, H, cfg.d_nope), dev)
    if cfg.d_rope > 0 or w_qr is not None:
        _need(w_qr, "w_qr", dt, (H * cfg.d_rope, K), dev)
    if cfg.d_rope > 0 or q_rope is not None:
        _need(q_rope, "q_rope", dt, (R, H, cfg.d_rope), dev)
    wp, wb = _ws(workspace, dev)
    check(lib.mla_project_inputs(cfg, B, n_new, dm, d_q, _ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(kv_norm_w),
                                 float(kv_norm_eps), _ptr(cache), _ptr(seq_off), _ptr(len_before), _ptr(w_dq),
                                 _ptr(w_uq), _ptr(w_qr), _ptr(q_nope), _ptr(q_rope), wp, wb, _stream(q_nope)),
          "mla_project_inputs")


def mla_prefill_explicit_workspace_size(cfg: MlaConfig, batch: int, n_q: int, max_seq_len: int) -> int:
    return int(lib.mla_prefill_explicit_workspace_size(cfg, batch, n_q, max_seq_len))


def mla_prefill_explicit(cfg: MlaConfig, q_nope: torch.Tensor, q_rope: torch.Tensor, cache: torch.Tensor,
                         seq_off: torch.Tensor, seq_len: torch.Tensor, max_seq_len: int, w_uk: torch.Tensor,
                         w_uv: torch.Tensor, o: torch.Tensor, lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, w_o: Optional[torch.Tensor] = None,
                         u: Optional[torch.Tensor] = None) -> None:
    """Non-absorbed attention of q [batch, n_q, H, .] over the cache; writes the heads' outputs
    o [batch, n_q, H, d_v] (and lse); with w_o [d_model, H * d_v] and u [batch * n_q, d_model] also
    u = W_O concat_i(o_i)."""
    dt = storage_dtype(cfg)
    H = cfg.n_heads
    if q_nope.dim() != 4:
        raise ValueError("q_nope must be [batch, n_q, H, d_nope]")
    B, n_q = q_nope.shape[0], q_nope.shape[1]
    dev = q_nope.device
    _need(q_nope, "q_nope", dt, (B, n_q, H, cfg.d_nope))
    _need(q_rope, "q_rope", dt, (B, n_q, H, cfg.d_rope), dev)
    _need(cache, "cache", dt, None, dev)
    _need(seq_off, "seq_off", torch.int64, (B,), dev)
    _need(seq_len, "seq_len", torch.int32, (B,), dev)
    _need(w_uk, "w_uk", dt, (H, cfg.d_nope, cfg.d_latent), dev)
    _need(w_uv, "w_uv", dt, (H, cfg.d_v, cfg.d_latent), dev)
    _need(o, "o", dt, (B, n_q, H, cfg.d_v), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, n_q, H), dev)
    if (w_o is None) != (u is None):
        raise ValueError("pass w_o and u together")
    d_model = 0
    if w_o is not None:
        if w_o.dim() != 2:
            raise ValueError("w_o must be [d_model, n_heads * d_v]")
        d_model = w_o.shape[0]
        _need(w_o, "w_o", dt, (d_model, H * cfg.d_v), dev)
        _need(u, "u", dt, (B * n_q, d_model), dev)
    wp, wb = _ws(workspace, dev)
    check(lib.mla_prefill_explicit(cfg, B, n_q, _ptr(q_nope), _ptr(q_rope), _ptr(cache), _ptr(seq_off), _ptr(seq_len),
                                   int(max_seq_len), _ptr(w_uk), _ptr(w_uv), wp, wb, _ptr(o), _ptr(lse), d_model,
                                   _ptr(w_o), _ptr(u), _stream(o)),
          "mla_prefill_explicit")


def mla_prefill_prefers_explicit(cfg: MlaConfig, batch: int, n_q: int, max_seq_len: int) -> bool:
    """True when the library would run n_q new query rows per sequence faster in the explicit form."""
    return bool(lib.mla_prefill_prefers_explicit(cfg, int(batch), int(n_q), int(max_seq_len)))


def mla_decode_advance(n_new: int, len_before: Optional[torch.Tensor] = None, seq_len: Optional[torch.Tensor] = None,
                       q_pos: Optional[torch.Tensor] = None) -> None:
    """len_before += n_new, seq_len += n_new, q_pos += n_new on the device (any may be None)."""
    given = [t for t in (len_before, seq_len, q_pos) if t is not None]
    if not given:
        return
    dev = given[0].device
    B = None
    for name, t in (("len_before", len_before), ("seq_len", seq_len)):
        if t is not None:
            _need(t, name, torch.int32, None, dev)
            if t.dim() != 1 or (B is not None and t.shape[0] != B):
                raise ValueError("len_before and seq_len must be [batch]")
            B = t.shape[0]
    R = 0
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, None, dev)
        if q_pos.dim() != 1:
            raise ValueError("q_pos must be [n_rows]")
        R = q_pos.shape[0]
    check(lib.mla_decode_advance(B or 0, int(n_new), _ptr(len_before), _ptr(seq_len), R, _ptr(q_pos),
                                 _stream(given[0])), "mla_decode_advance")


def version() -> str:
    return lib.mla_version().decode()


__all__ = [
    "make_config",
    "storage_dtype",
    "mla_rope_append",
    "mla_absorb_q",
    "mla_decode_attn_workspace_size",
    "mla_decode_step_workspace_size",
    "mla_decode_step",
    "mla_decode_attn",
    "mla_out_proj",
    "mla_project_workspace_size",
    "mla_project_kv_append",
    "mla_project_q",
    "mla_project_inputs_workspace_size",
    "mla_project_inputs",
    "mla_decode_advance",
    "mla_prefill_explicit_workspace_size",
    "mla_prefill_explicit",
    "version",
    "_lib",
]
