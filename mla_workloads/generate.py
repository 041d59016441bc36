"""Seeded input generators.

Every tensor has its own independent stream,
``numpy.random.default_rng(SeedSequence([config_id, tensor_id, *index]))``, so a
tensor does not depend on which other tensors were drawn or in what order.
Values are drawn in float32 and rounded once (round-to-nearest-even) to the
configuration's storage dtype. Returned arrays are float32 holding exactly the
storage values; callers upcast (oracle) or reinterpret (device upload).

Distribution recipe (the input distribution, not the method):
  * weights W ~ N(0, 1/fan_in), with fan_in the input width of the
    ``nn.Linear`` the weight belongs to (``[out, in]`` layout);
  * hidden states, unrotated position keys/queries and content queries ~ N(0, 1);
  * cache-side latent rows: N(0, I) rows scaled to unit RMS (eps 1e-6) when the
    configuration says the latent is RMS-normalised, plain N(0, 1) otherwise.
"""

from __future__ import annotations

import enum
from typing import Dict, Optional

import numpy as np

from .configs import MLAConfig


class TensorId(enum.IntEnum):
    H = 1
    W_DKV = 2
    W_KR = 3
    W_Q = 4
    W_QR = 5
    W_UK = 6
    W_UV = 7
    W_O = 8
    C = 9
    K_ROPE = 10
    Q_NOPE = 11
    Q_ROPE = 12
    LENGTHS = 13
    W_DQ = 14
    W_UQ = 15
    KV_NORM = 16


def _rng(cfg: MLAConfig, tid: TensorId, *index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cfg.cid), int(tid), *[int(i) for i in index]]))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bfloat16 (ties to even); returns float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    r = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).reshape(f.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of float32 values that are already bf16-representable."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bfloat16-representable; call round_bf16 first")
    return (u >> 16).astype(np.uint16)


def _store(cfg: MLAConfig, x: np.ndarray) -> np.ndarray:
    if cfg.dtype == "bf16":
        return round_bf16(x)
    if cfg.dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown storage dtype {cfg.dtype!r}")


def _normal(cfg: MLAConfig, tid: TensorId, shape, std: float = 1.0, *index: int) -> np.ndarray:
    g = _rng(cfg, tid, *index).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        g *= np.float32(std)
    return g


def seq_lens(cfg: MLAConfig) -> np.ndarray:
    """Keys per sequence, counting the n_q new tokens (int64 [batch])."""
    if cfg.fixed_len is not None:
        return np.full(cfg.batch, cfg.fixed_len, dtype=np.int64)
    lo, hi = cfg.ragged_range
    hist = _rng(cfg, TensorId.LENGTHS).integers(lo, hi, size=cfg.batch, endpoint=True)
    return (hist + cfg.n_q).astype(np.int64)


def cache_latent(cfg: MLAConfig, b: int, n: Optional[int] = None) -> np.ndarray:
    """Latent rows c for every token of sequence b: float32 [n_b, d_latent]."""
    if n is None:
        n = int(seq_lens(cfg)[b])
    g = _normal(cfg, TensorId.C, (n, cfg.d_latent), 1.0, b)
    if cfg.latent_rms_norm:
        g64 = g.astype(np.float64)
        g = (g64 / np.sqrt(np.mean(g64 * g64, axis=-1, keepdims=True) + 1e-6)).astype(np.float32)
    return _store(cfg, g)


def cache_rope_pre(cfg: MLAConfig, b: int, n: Optional[int] = None) -> np.ndarray:
    """Unrotated shared position keys for every token of sequence b: float32 [n_b, d_rope]."""
    if n is None:
        n = int(seq_lens(cfg)[b])
    return _store(cfg, _normal(cfg, TensorId.K_ROPE, (n, cfg.d_rope), 1.0, b))


def query_nope(cfg: MLAConfig, b: int) -> np.ndarray:
    """Content queries of sequence b's new tokens: float32 [n_q, H, d_nope]."""
    return _store(cfg, _normal(cfg, TensorId.Q_NOPE, (cfg.n_q, cfg.n_heads, cfg.d_nope), 1.0, b))


def query_rope_pre(cfg: MLAConfig, b: int) -> np.ndarray:
    """Unrotated per-head position queries of sequence b's new tokens: float32 [n_q, H, d_rope]."""
    return _store(cfg, _normal(cfg, TensorId.Q_ROPE, (cfg.n_q, cfg.n_heads, cfg.d_rope), 1.0, b))


def weight_uk(cfg: MLAConfig) -> np.ndarray:
    """W_UK viewed per head: float32 [H, d_nope, d_latent] (nn.Linear(d_latent, H*d_nope).weight)."""
    return _store(cfg, _normal(cfg, TensorId.W_UK, (cfg.n_heads, cfg.d_nope, cfg.d_latent),
                               1.0 / np.sqrt(cfg.d_latent)))


def weight_uv(cfg: MLAConfig) -> np.ndarray:
    """W_UV viewed per head: float32 [H, d_v, d_latent] (nn.Linear(d_latent, H*d_v).weight)."""
    return _store(cfg, _normal(cfg, TensorId.W_UV, (cfg.n_heads, cfg.d_v, cfg.d_latent),
                               1.0 / np.sqrt(cfg.d_latent)))


def weight_o(cfg: MLAConfig) -> np.ndarray:
    """W_O: float32 [d_model, H*d_v] (nn.Linear(H*d_v, d_model).weight)."""
    fan_in = cfg.n_heads * cfg.d_v
    return _store(cfg, _normal(cfg, TensorId.W_O, (cfg.d_model, fan_in), 1.0 / np.sqrt(fan_in)))


def full_layer_inputs(cfg: MLAConfig, n_tokens: int) -> Dict[str, np.ndarray]:
    """Hidden states and every projection weight of one layer, for whole-layer checks.

    Keys: h [n, d_model]; w_dkv [d_latent, d_model]; w_kr [d_rope, d_model];
    either w_q [H*d_nope, d_model] (no query compression) or w_dq [q_lora, d_model]
    and w_uq [H*d_nope, q_lora]; w_qr [H*d_rope, d_model or q_lora];
    w_uk, w_uv per head; w_o; and, when the configuration RMS-normalises the latent,
    kv_norm_w [d_latent] ~ 1 + 0.25 N(0, 1) (a trained-looking gain rather than the
    all-ones initial value, so that a dropped gain shows).
    """
    H, dm = cfg.n_heads, cfg.d_model
    out = {
        "h": _store(cfg, _normal(cfg, TensorId.H, (n_tokens, dm))),
        "w_dkv": _store(cfg, _normal(cfg, TensorId.W_DKV, (cfg.d_latent, dm), 1.0 / np.sqrt(dm))),
        "w_kr": _store(cfg, _normal(cfg, TensorId.W_KR, (cfg.d_rope, dm), 1.0 / np.sqrt(dm))),
        "w_uk": weight_uk(cfg),
        "w_uv": weight_uv(cfg),
        "w_o": weight_o(cfg),
    }
    if cfg.latent_rms_norm:
        out["kv_norm_w"] = _store(cfg, 1.0 + _normal(cfg, TensorId.KV_NORM, (cfg.d_latent,), 0.25))
    if cfg.q_lora is None:
        out["w_q"] = _store(cfg, _normal(cfg, TensorId.W_Q, (H * cfg.d_nope, dm), 1.0 / np.sqrt(dm)))
        out["w_qr"] = _store(cfg, _normal(cfg, TensorId.W_QR, (H * cfg.d_rope, dm), 1.0 / np.sqrt(dm)))
    else:
        ql = cfg.q_lora
        out["w_dq"] = _store(cfg, _normal(cfg, TensorId.W_DQ, (ql, dm), 1.0 / np.sqrt(dm)))
        out["w_uq"] = _store(cfg, _normal(cfg, TensorId.W_UQ, (H * cfg.d_nope, ql), 1.0 / np.sqrt(ql)))
        out["w_qr"] = _store(cfg, _normal(cfg, TensorId.W_QR, (H * cfg.d_rope, ql), 1.0 / np.sqrt(ql)))
    return out
