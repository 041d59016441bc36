"""Helpers shared by the GPU tests: upload seeded inputs, run the four C-ABI calls,
and compare with the oracle. Imported only by tests."""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import mla_decode_decoupled_amd as mla
from mla_workloads import MLAConfig
from mla_workloads import generate as G


def lib_config(cfg: MLAConfig, scale: Optional[float] = None):
    return mla.make_config(cfg.n_heads, cfg.d_nope, cfg.d_latent, cfg.d_rope, cfg.d_v, cfg.dtype,
                           cfg.rope_base, cfg.softmax_scale if scale is None else scale)


def tdev(x: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(dtype)


@dataclass
class HostInputs:
    cfg: MLAConfig
    lens: np.ndarray                  # keys per sequence incl. the n_q new tokens
    c: List[np.ndarray]               # per sequence [n_b, d_latent]
    k_pre: List[np.ndarray]           # per sequence [n_b, d_rope] unrotated
    q_nope: np.ndarray                # [B, n_q, H, d_nope]
    q_rope: np.ndarray                # [B, n_q, H, d_rope] unrotated
    w_uk: np.ndarray
    w_uv: np.ndarray


def host_inputs(cfg: MLAConfig, lens: Optional[Sequence[int]] = None) -> HostInputs:
    lens = G.seq_lens(cfg) if lens is None else np.asarray(lens, dtype=np.int64)
    B = len(lens)
    return HostInputs(
        cfg=cfg, lens=lens,
        c=[G.cache_latent(cfg, b, int(lens[b])) for b in range(B)],
        k_pre=[G.cache_rope_pre(cfg, b, int(lens[b])) for b in range(B)],
        q_nope=np.stack([G.query_nope(cfg, b) for b in range(B)]),
        q_rope=np.stack([G.query_rope_pre(cfg, b) for b in range(B)]),
        w_uk=G.weight_uk(cfg), w_uv=G.weight_uv(cfg),
    )


@dataclass
class DeviceRun:
    cache: torch.Tensor
    seq_off: torch.Tensor
    seq_len: torch.Tensor
    q_packed: torch.Tensor
    z: torch.Tensor
    lse: torch.Tensor
    o: torch.Tensor


def run_pipeline(hi: HostInputs, n_splits: int = 0, scale: Optional[float] = None,
                 lib_cfg=None, max_len: Optional[int] = None) -> DeviceRun:
    """Cache the history, then one step: append the n_q new tokens, absorb, attend, project."""
    cfg = hi.cfg
    lc = lib_config(cfg, scale) if lib_cfg is None else lib_cfg
    dt = mla.storage_dtype(lc)
    B, n_q, H = len(hi.lens), cfg.n_q, cfg.n_heads
    lens = hi.lens
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    cache = torch.empty((int(lens.sum()), cfg.row), dtype=dt, device="cuda")
    cache.fill_(float("nan"))                 # every row read must have been written
    seq_off = torch.from_numpy(offs).cuda()
    seq_len = torch.from_numpy(lens.astype(np.int32)).cuda()
    # history: tokens 0 .. n_b - n_q - 1 of every sequence
    for b in range(B):
        h = int(lens[b]) - n_q
        if h > 0:
            mla.mla_rope_append(lc, tdev(hi.c[b][None, :h], dt), tdev(hi.k_pre[b][None, :h], dt), cache,
                                seq_off[b:b + 1], torch.zeros(1, dtype=torch.int32, device="cuda"))
    # the step: append every sequence's n_q new tokens in one call
    c_new = np.stack([hi.c[b][int(lens[b]) - n_q:] for b in range(B)])
    k_new = np.stack([hi.k_pre[b][int(lens[b]) - n_q:] for b in range(B)])
    len_before = torch.from_numpy((lens - n_q).astype(np.int32)).cuda()
    mla.mla_rope_append(lc, tdev(c_new, dt), tdev(k_new, dt), cache, seq_off, len_before)
    # absorb: rows are (b, t) flattened; positions n_b - n_q + t
    R = B * n_q
    q_pos = torch.from_numpy(np.concatenate([np.arange(int(lens[b]) - n_q, int(lens[b])) for b in range(B)])
                             .astype(np.int32)).cuda()
    q_packed = torch.empty((R, H, cfg.row), dtype=dt, device="cuda")
    mla.mla_absorb_q(lc, tdev(hi.q_nope.reshape(R, H, cfg.d_nope), dt),
                     tdev(hi.q_rope.reshape(R, H, cfg.d_rope), dt), q_pos, tdev(hi.w_uk, dt), q_packed)
    z = torch.empty((B, n_q, H, cfg.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device="cuda")
    max_len = int(lens.max()) if max_len is None else int(max_len)
    ws_bytes = mla.mla_decode_attn_workspace_size(lc, B, n_q, max_len, n_splits)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    mla.mla_decode_attn(lc, q_packed.view(B, n_q, H, cfg.row), cache, seq_off, seq_len, max_len, z, lse,
                        n_splits=n_splits, workspace=ws)
    o = torch.empty((R, H, cfg.d_v), dtype=dt, device="cuda")
    mla.mla_out_proj(lc, z.view(R, H, cfg.d_latent), tdev(hi.w_uv, dt), o)
    torch.cuda.synchronize()
    return DeviceRun(cache, seq_off, seq_len, q_packed.view(B, n_q, H, cfg.row), z, lse, o.view(B, n_q, H, cfg.d_v))


def run_step(hi: HostInputs, n_splits: int = 0, scale: Optional[float] = None, lib_cfg=None,
             max_len: Optional[int] = None, noalloc: bool = False) -> DeviceRun:
    """The same history and step as run_pipeline, the step as one mla_decode_step call (or, with
    noalloc, one mla_decode_step_noalloc call, which brings its own scratch)."""
    cfg = hi.cfg
    lc = lib_config(cfg, scale) if lib_cfg is None else lib_cfg
    dt = mla.storage_dtype(lc)
    B, n_q, H = len(hi.lens), cfg.n_q, cfg.n_heads
    lens = hi.lens
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    cache = torch.empty((int(lens.sum()), cfg.row), dtype=dt, device="cuda")
    cache.fill_(float("nan"))
    seq_off = torch.from_numpy(offs).cuda()
    seq_len = torch.from_numpy(lens.astype(np.int32)).cuda()
    for b in range(B):
        h = int(lens[b]) - n_q
        if h > 0:
            mla.mla_rope_append(lc, tdev(hi.c[b][None, :h], dt), tdev(hi.k_pre[b][None, :h], dt), cache,
                                seq_off[b:b + 1], torch.zeros(1, dtype=torch.int32, device="cuda"))
    c_new = tdev(np.stack([hi.c[b][int(lens[b]) - n_q:] for b in range(B)]), dt)
    k_new = tdev(np.stack([hi.k_pre[b][int(lens[b]) - n_q:] for b in range(B)]), dt)
    R = B * n_q
    q_packed = torch.empty((R, H, cfg.row), dtype=dt, device="cuda")
    z = torch.empty((B, n_q, H, cfg.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device="cuda")
    o = torch.empty((R, H, cfg.d_v), dtype=dt, device="cuda")
    max_len = int(lens.max()) if max_len is None else int(max_len)
    qn, qr = tdev(hi.q_nope.reshape(R, H, cfg.d_nope), dt), tdev(hi.q_rope.reshape(R, H, cfg.d_rope), dt)
    wuk, wuv = tdev(hi.w_uk, dt), tdev(hi.w_uv, dt)
    if noalloc:
        mla.mla_decode_step_noalloc(lc, c_new, k_new, qn, qr, wuk, wuv, cache, seq_off, seq_len, max_len, q_packed, z,
                                    o, lse=lse, n_splits=n_splits)
    else:
        ws = torch.empty(mla.mla_decode_step_workspace_size(lc, B, n_q, max_len, n_splits), dtype=torch.uint8,
                         device="cuda")
        mla.mla_decode_step(lc, c_new, k_new, qn, qr, wuk, wuv, cache, seq_off, seq_len, max_len, q_packed, z, o,
                            lse=lse, n_splits=n_splits, workspace=ws)
    torch.cuda.synchronize()
    return DeviceRun(cache, seq_off, seq_len, q_packed.view(B, n_q, H, cfg.row), z, lse, o.view(B, n_q, H, cfg.d_v))


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str,
                 abs_tol: Optional[float] = None, rel_l2: Optional[float] = None) -> Dict[str, float]:
    """The parity bar: fp32 -> max|err| <= 1e-5; bf16 -> max|err| <= 2e-2 and rel-L2 <= 1e-2."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    max_err = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ref)) or 1.0
    rel = float(np.linalg.norm(got - ref)) / denom
    if dtype == "f32":
        a = 1e-5 if abs_tol is None else abs_tol
        assert max_err <= a, f"{what}: max|err| {max_err:.3e} > {a:.1e}"
    else:
        a = 2e-2 if abs_tol is None else abs_tol
        r = 1e-2 if rel_l2 is None else rel_l2
        assert max_err <= a, f"{what}: max|err| {max_err:.3e} > {a:.1e} (rel-L2 {rel:.2e})"
        assert rel <= r, f"{what}: rel-L2 {rel:.3e} > {r:.1e} (max|err| {max_err:.2e})"
    return {"max_err": max_err, "rel_l2": rel}
