"""Multi-step, multi-layer decode loop over the library's calls.

A stack of MLA attention layers is run token by token the way the pages run their check of the
absorbed form ("从零理解 MLA", the decode loop after the decoupled-RoPE code: every step appends
the new token's latent and rotated position key to the cache, then attends over the grown
cache): per layer, mla_project_inputs (mla_project_kv_append and mla_project_q in one call) ->
mla_absorb_q -> mla_decode_attn -> mla_out_proj (with W_O), and the layer's output u is the next
layer's input (the residual stream and the feed-forward blocks of a full model are not part of
this stack). A step of many new tokens per sequence (a prefill chunk) takes the explicit form
instead, mla_project_inputs -> mla_prefill_explicit (with W_O), whenever the library reports it as
the faster one for that row count (mla_prefill_prefers_explicit; "Decoupled RoPE · MLA Part 2", §5
closing remark: absorption is the decode form). After the last layer, mla_decode_advance moves
every position on by the tokens just appended, so one recorded decode step — a HIP graph captured
through torch — can be replayed for every following token. The attention's split plan is chosen
from the cache capacity (the grid bound every step shares), not from the current length, so one
captured step serves every following token.

This module only allocates buffers, sets positions and enqueues library calls; every step of the
computation runs in libmla's kernels.
"""

from __future__ import annotations

from typing import Dict, List, Optional

import torch

from . import ops
from ._lib import MlaConfig


class _StepBuffers:
    """Device buffers of one step shape (batch x n_new tokens)."""

    def __init__(self, stack: "DecodeStack", n_new: int):
        cfg, B, dev, dt = stack.cfg, stack.batch, stack.device, stack.dtype
        R = B * n_new
        H = cfg.n_heads
        self.n_new = n_new
        self.len_before = torch.zeros(B, dtype=torch.int32, device=dev)
        self.seq_len = torch.zeros(B, dtype=torch.int32, device=dev)
        self.q_pos = torch.zeros(R, dtype=torch.int32, device=dev)
        self.q_nope = torch.empty((R, H, cfg.d_nope), dtype=dt, device=dev)
        self.q_rope = torch.empty((R, H, cfg.d_rope), dtype=dt, device=dev)
        self.q_packed = torch.empty((B, n_new, H, cfg.d_latent + cfg.d_rope), dtype=dt, device=dev)
        self.z = torch.empty((B, n_new, H, cfg.d_latent), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, n_new, H), dtype=torch.float32, device=dev)
        self.o = torch.empty((R, H, cfg.d_v), dtype=dt, device=dev)
        # layer outputs ping-pong: layer l writes u[l % 2], layer l + 1 reads it
        self.u = [torch.empty((B, n_new, stack.d_model), dtype=dt, device=dev) for _ in range(2)]
        self.h_in = torch.empty((B, n_new, stack.d_model), dtype=dt, device=dev)
        pw = ops.mla_project_inputs_workspace_size(cfg, R, stack.d_model, stack.d_q)
        self.ws_proj = torch.empty(max(pw, 256), dtype=torch.uint8, device=dev)
        # the explicit form for long chunks when the library prefers it, else the absorbed calls
        self.explicit = ops.mla_prefill_prefers_explicit(cfg, B, n_new, stack.capacity)
        if self.explicit:
            xw = ops.mla_prefill_explicit_workspace_size(cfg, B, n_new, stack.capacity)
            self.ws_attn = torch.empty(max(xw, 256), dtype=torch.uint8, device=dev)
        else:
            aw = ops.mla_decode_attn_workspace_size(cfg, B, n_new, stack.capacity, stack.n_splits)
            self.ws_attn = torch.empty(max(aw, 256), dtype=torch.uint8, device=dev)

    def set_positions(self, length: int) -> None:
        """Positions of a step that appends n_new tokens after `length` cached ones."""
        n = self.n_new
        self.len_before.fill_(length)
        self.seq_len.fill_(length + n)
        self.q_pos.copy_((torch.arange(n, dtype=torch.int32, device=self.q_pos.device) + length)
                         .repeat(self.len_before.shape[0]))


class DecodeStack:
    """n_layers MLA attention layers with one cache each, for `batch` sequences of equal length.

    layers[l] holds device tensors in the storage dtype: w_dkv [d_latent, d_model], w_kr
    [d_rope, d_model], optional kv_norm_w [d_latent], optional w_dq [d_q, d_model], w_uq
    [H d_nope, d_q or d_model], w_qr [H d_rope, d_q or d_model], w_uk [H, d_nope, d_latent],
    w_uv [H, d_v, d_latent], w_o [d_model, H d_v]. Each cache holds `capacity` tokens per sequence.
    """

    def __init__(self, cfg: MlaConfig, layers: List[Dict[str, torch.Tensor]], batch: int, capacity: int,
                 kv_norm_eps: float = 1e-6, n_splits: int = 0):
        if not layers:
            raise ValueError("need at least one layer")
        self.cfg = cfg
        self.layers = layers
        self.batch = int(batch)
        self.capacity = int(capacity)
        self.kv_norm_eps = float(kv_norm_eps)
        self.n_splits = int(n_splits)
        w0 = layers[0]
        self.device = w0["w_dkv"].device
        self.dtype = ops.storage_dtype(cfg)
        self.d_model = int(w0["w_dkv"].shape[1])
        self.d_q = int(w0["w_dq"].shape[0]) if w0.get("w_dq") is not None else 0
        row = cfg.d_latent + cfg.d_rope
        self.caches = [torch.empty((self.batch * self.capacity, row), dtype=self.dtype, device=self.device)
                       for _ in layers]
        self.seq_off = torch.arange(self.batch, dtype=torch.int64, device=self.device) * self.capacity
        self.length = 0          # tokens cached per sequence
        self._bufs: Dict[int, _StepBuffers] = {}
        self.last_prefill_path: Optional[str] = None   # "explicit" or "absorbed": the form of the last forward()

    def buffers(self, n_new: int) -> _StepBuffers:
        if n_new not in self._bufs:
            self._bufs[n_new] = _StepBuffers(self, n_new)
        return self._bufs[n_new]

    def _enqueue(self, b: _StepBuffers) -> torch.Tensor:
        """All layers of one step on the current stream, then the position advance; returns the
        last layer's output buffer."""
        cfg, B, n = self.cfg, self.batch, b.n_new
        R = B * n
        x = b.h_in
        H = cfg.n_heads
        for l, w in enumerate(self.layers):
            ops.mla_project_inputs(cfg, x, w["w_dkv"], w["w_kr"], self.caches[l], self.seq_off, b.len_before,
                                   w["w_uq"], w["w_qr"], b.q_nope, b.q_rope, w_dq=w.get("w_dq"),
                                   kv_norm_w=w.get("kv_norm_w"), kv_norm_eps=self.kv_norm_eps, workspace=b.ws_proj)
            u = b.u[l % 2]
            if b.explicit:
                ops.mla_prefill_explicit(cfg, b.q_nope.view(B, n, H, cfg.d_nope), b.q_rope.view(B, n, H, cfg.d_rope),
                                         self.caches[l], self.seq_off, b.seq_len, self.capacity, w["w_uk"], w["w_uv"],
                                         b.o.view(B, n, H, cfg.d_v), b.lse, workspace=b.ws_attn, w_o=w["w_o"],
                                         u=u.view(R, self.d_model))
                x = u
                continue
            ops.mla_absorb_q(cfg, b.q_nope, b.q_rope, b.q_pos, w["w_uk"], b.q_packed.view(R, cfg.n_heads, -1))
            ops.mla_decode_attn(cfg, b.q_packed, self.caches[l], self.seq_off, b.seq_len, self.capacity, b.z, b.lse,
                                n_splits=self.n_splits, workspace=b.ws_attn)
            ops.mla_out_proj(cfg, b.z.view(R, cfg.n_heads, cfg.d_latent), w["w_uv"], b.o, w_o=w["w_o"],
                             u=u.view(R, self.d_model))
            x = u
        ops.mla_decode_advance(n, len_before=b.len_before, seq_len=b.seq_len, q_pos=b.q_pos)
        return x

    def forward(self, h: torch.Tensor) -> torch.Tensor:
        """Append h [batch, n_new, d_model] (n_new >= 1 tokens per sequence, causal among
        themselves) to every layer and return the last layer's output [batch, n_new, d_model]
        (a view of an internal buffer, valid until the next call with the same n_new)."""
        if h.dim() != 3 or h.shape[0] != self.batch or h.shape[2] != self.d_model:
            raise ValueError(f"h must be [{self.batch}, n_new, {self.d_model}]")
        n = int(h.shape[1])
        if self.length + n > self.capacity:
            raise ValueError(f"cache capacity {self.capacity} exceeded")
        b = self.buffers(n)
        b.set_positions(self.length)
        b.h_in.copy_(h)
        out = self._enqueue(b)
        self.last_prefill_path = "explicit" if b.explicit else "absorbed"
        self.length += n
        return out

    def capture_decode(self) -> "DecodeGraph":
        """Record one decode step (one token per sequence through every layer) as a HIP graph."""
        return DecodeGraph(self)


class DecodeGraph:
    """A captured one-token step of a DecodeStack. Write the next token's hidden states into
    `h_in`, call replay(), read `u`. Positions advance on the device inside the graph; the
    stack's host-side length follows."""

    def __init__(self, stack: DecodeStack):
        self.stack = stack
        self.bufs = stack.buffers(1)
        self.bufs.set_positions(stack.length)
        self.h_in = self.bufs.h_in
        torch.cuda.synchronize(stack.device)
        self.graph = torch.cuda.CUDAGraph()
        # capturing enqueues nothing that runs; the positions set above are still the next step's
        with torch.cuda.graph(self.graph):
            self.u = stack._enqueue(self.bufs)

    def replay(self) -> torch.Tensor:
        st = self.stack
        if st.length + 1 > st.capacity:
            raise ValueError(f"cache capacity {st.capacity} exceeded")
        self.graph.replay()
        st.length += 1
        return self.u


def random_layers(cfg: MlaConfig, n_layers: int, d_model: int, d_q: int, device, seed: int = 0,
                  kv_norm: bool = True) -> List[Dict[str, torch.Tensor]]:
    """Seeded random layer weights on the device, W ~ N(0, 1/fan_in) in the storage dtype (for
    timing runs; the parity tests upload the seeded host generators' weights instead)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = ops.storage_dtype(cfg)
    H = cfg.n_heads

    def w(shape, fan_in):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) / fan_in ** 0.5).to(dt)

    layers = []
    for _ in range(n_layers):
        K = d_q if d_q > 0 else d_model
        lw = {
            "w_dkv": w((cfg.d_latent, d_model), d_model),
            "w_kr": w((cfg.d_rope, d_model), d_model),
            "w_uq": w((H * cfg.d_nope, K), K),
            "w_qr": w((H * cfg.d_rope, K), K),
            "w_uk": w((H, cfg.d_nope, cfg.d_latent), cfg.d_latent),
            "w_uv": w((H, cfg.d_v, cfg.d_latent), cfg.d_latent),
            "w_o": w((d_model, H * cfg.d_v), H * cfg.d_v),
        }
        if d_q > 0:
            lw["w_dq"] = w((d_q, d_model), d_model)
        if kv_norm:
            lw["kv_norm_w"] = (1.0 + 0.25 * torch.randn((cfg.d_latent,), generator=g, device=device)).to(dt)
        layers.append(lw)
    return layers


__all__ = ["DecodeStack", "DecodeGraph", "random_layers"]
