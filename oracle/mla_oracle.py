"""Plain fp64 CPU oracle for Multi-head Latent Attention with decoupled RoPE.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module. It shares no code with the HIP path and
imports nothing from it; it works on numpy arrays given to it by the caller.

What it computes, and where the pages define it:

* RoPE: each consecutive pair (x_2j, x_2j+1) of a position vector at position p
  is turned by the angle p * theta_j, theta_j = base^(-2j/d)
  ("Decoupled RoPE · MLA Part 2", §4 rotation rule and the ``rope`` helper of §7;
  the block-diagonal R_n of "旋转约束下的压缩：从 RoPE 到 DeepSeek MLA",
  section "数学证明"). A half-split pairing (j, j + d/2), used by the code of
  "从零理解 MLA" (section "解耦 RoPE"), is available by flag.
* Non-absorbed attention, the oracle's method: per head the content key
  K_C = C W_UK,i^T and the value V = C W_UV,i^T are rebuilt explicitly
  ("Decoupled RoPE · MLA Part 2", §2.1 first fallback and ``forward_naive`` in §7),
  the shared rotated position key is concatenated to every head's key (§3.2, §3.3),
  the query is [q_C ; RoPE(q_R)], scores are scaled by 1/sqrt(d_h + d_R) (§4.6 note),
  causally masked with the diagonal offset S - L used when a cache is present
  ("从零理解 MLA", section "KV Cache", code example and the remark after it),
  softmaxed, and o = alpha V; u = W_O concat_i(o_i).
* Diagnostics used to check the absorbed calls one at a time: the latent aggregate
  z = alpha C (so o = W_UV,i z by associativity: "从零理解 MLA", section "矩阵吸收",
  output-side equation) and the natural-log LSE of the scaled, masked scores.
* The absorbed form (q~ = W_UK,i^T q_C, scores against packed [c ; k_R] rows,
  z = alpha C, o = W_UV,i z; "Decoupled RoPE · MLA Part 2" §5 and
  ``forward_absorbed``; "从零理解 MLA" ``absorbed_step``) exists here only so the
  tests can show it equals the explicit form, and to define each absorbed call's
  output (q_packed, cache rows) in isolation.

Everything is float64. Inputs are upcast from whatever the caller passes.
"""

from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence

import numpy as np

_F = np.float64


# --------------------------------------------------------------------------- RoPE
def rope_inv_freq(d_rope: int, base: float) -> np.ndarray:
    """theta_j = base^(-2j/d_rope), j = 0 .. d_rope/2 - 1."""
    if d_rope % 2:
        raise ValueError("RoPE width must be even")
    j = np.arange(d_rope // 2, dtype=_F)
    return np.power(_F(base), -2.0 * j / d_rope)


def rope_rotate(x, positions, base: float, layout: str = "interleaved") -> np.ndarray:
    """Rotate the last axis of ``x`` by position.

    ``positions`` must broadcast against ``x.shape[:-1]``. Pair j is turned by
    positions * theta_j: [a cos - b sin, a sin + b cos].
    """
    x = np.asarray(x, dtype=_F)
    d = x.shape[-1]
    if d == 0:
        return x.copy()
    ang = np.asarray(positions, dtype=_F)[..., None] * rope_inv_freq(d, base)
    cos, sin = np.cos(ang), np.sin(ang)
    out = np.empty(np.broadcast_shapes(x.shape, cos.shape[:-1] + (d,)), dtype=_F)
    if layout == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * cos - b * sin
        out[..., 1::2] = a * sin + b * cos
    elif layout == "half":
        h = d // 2
        a, b = x[..., :h], x[..., h:]
        out[..., :h] = a * cos - b * sin
        out[..., h:] = a * sin + b * cos
    else:
        raise ValueError(f"unknown RoPE layout {layout!r}")
    return out


# ---------------------------------------------------------------- masking/softmax
def visible(n_keys: int, n_q: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean [len(rows), n_keys]: query row t sees key j iff j <= n_keys - n_q + t."""
    t = np.arange(n_q) if rows is None else np.asarray(rows)
    j = np.arange(n_keys)
    return j[None, :] <= (n_keys - n_q + t)[:, None]


def softmax_masked(x: np.ndarray, vis: np.ndarray):
    """Row softmax over visible entries; returns (alpha, lse) with lse the natural log-sum-exp."""
    x = np.where(vis, x, -np.inf)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    s = np.sum(e, axis=-1, keepdims=True)
    return e / s, (m + np.log(s))[..., 0]


# ------------------------------------------------------------- explicit (oracle)
def explicit_attention(
    c,
    k_rope_pre,
    q_nope,
    q_rope_pre,
    w_uk,
    w_uv,
    *,
    scale: float,
    base: float,
    pos_offset: int = 0,
    heads: Optional[Iterable[int]] = None,
    rows: Optional[Iterable[int]] = None,
    layout: str = "interleaved",
    keep_scores: bool = False,
) -> Dict[str, np.ndarray]:
    """Non-absorbed MLA attention for one sequence.

    c [n, d_c] latent of every key token; k_rope_pre [n, d_R] unrotated shared
    position keys; q_nope [n_q, H, d_nope]; q_rope_pre [n_q, H, d_R] unrotated;
    w_uk [H, d_nope, d_c]; w_uv [H, d_v, d_c]. Key j sits at position
    pos_offset + j; query row t at pos_offset + n - n_q + t.

    Returns (over the selected rows r and heads h, in the given order):
      o [r, h, d_v], z [r, h, d_c] (= alpha C), lse [r, h],
      k_rot [n, d_R], q_rot [r, h, d_R],
      and with keep_scores also logits [r, h, n] (scaled, masked) and alpha [r, h, n].
    """
    c = np.asarray(c, dtype=_F)
    k_rope_pre = np.asarray(k_rope_pre, dtype=_F)
    q_nope = np.asarray(q_nope, dtype=_F)
    q_rope_pre = np.asarray(q_rope_pre, dtype=_F)
    w_uk = np.asarray(w_uk, dtype=_F)
    w_uv = np.asarray(w_uv, dtype=_F)
    n = c.shape[0]
    n_q, H = q_nope.shape[0], q_nope.shape[1]
    rows = np.arange(n_q) if rows is None else np.asarray(list(rows), dtype=np.int64)
    heads = np.arange(H) if heads is None else np.asarray(list(heads), dtype=np.int64)

    pos_k = pos_offset + np.arange(n, dtype=_F)
    pos_q = pos_offset + (n - n_q) + rows.astype(_F)
    k_rot = rope_rotate(k_rope_pre, pos_k, base, layout)                     # shared by all heads
    q_rot = rope_rotate(q_rope_pre[rows][:, heads], pos_q[:, None], base, layout)
    vis = visible(n, n_q, rows)

    R, NH = len(rows), len(heads)
    d_v = w_uv.shape[1]
    o = np.zeros((R, NH, d_v), dtype=_F)
    z = np.zeros((R, NH, c.shape[1]), dtype=_F)
    lse = np.zeros((R, NH), dtype=_F)
    logits_all = np.zeros((R, NH, n), dtype=_F) if keep_scores else None
    alpha_all = np.zeros((R, NH, n), dtype=_F) if keep_scores else None
    for hi, i in enumerate(heads):
        k_c = c @ w_uk[i].T                                   # [n, d_nope] rebuilt content keys
        v = c @ w_uv[i].T                                     # [n, d_v] rebuilt values
        k = np.concatenate([k_c, k_rot], axis=1)              # [n, d_nope + d_R]
        q = np.concatenate([q_nope[rows, i], q_rot[:, hi]], axis=1)
        x = scale * (q @ k.T)                                 # [R, n]
        alpha, l = softmax_masked(x, vis)
        o[:, hi] = alpha @ v
        z[:, hi] = alpha @ c
        lse[:, hi] = l
        if keep_scores:
            logits_all[:, hi] = np.where(vis, x, -np.inf)
            alpha_all[:, hi] = alpha
    out = {"o": o, "z": z, "lse": lse, "k_rot": k_rot, "q_rot": q_rot}
    if keep_scores:
        out["logits"] = logits_all
        out["alpha"] = alpha_all
    return out


def output_projection(o, w_o) -> np.ndarray:
    """u = W_O concat_i(o_i): o [r, H, d_v], w_o [d_model, H*d_v] -> [r, d_model]."""
    o = np.asarray(o, dtype=_F)
    return o.reshape(o.shape[0], -1) @ np.asarray(w_o, dtype=_F).T


# ------------------------------------------------------- absorbed-form pieces
def absorb_query(q_nope, w_uk) -> np.ndarray:
    """q~[r, i] = W_UK,i^T q_nope[r, i]: [r, H, d_nope] x [H, d_nope, d_c] -> [r, H, d_c]."""
    q_nope = np.asarray(q_nope, dtype=_F)
    w_uk = np.asarray(w_uk, dtype=_F)
    out = np.empty((q_nope.shape[0], q_nope.shape[1], w_uk.shape[2]), dtype=_F)
    for i in range(q_nope.shape[1]):
        out[:, i] = q_nope[:, i] @ w_uk[i]
    return out


def cache_rows(c, k_rope_pre, positions, base: float, layout: str = "interleaved") -> np.ndarray:
    """Packed cache rows [c ; RoPE_p(k_R)] for tokens at ``positions``: [n, d_c + d_R]."""
    c = np.asarray(c, dtype=_F)
    return np.concatenate([c, rope_rotate(k_rope_pre, np.asarray(positions, dtype=_F), base, layout)], axis=1)


def packed_query(q_nope, q_rope_pre, positions, w_uk, base: float, layout: str = "interleaved") -> np.ndarray:
    """[q~ ; RoPE_p(q_R)] per row and head: [r, H, d_c + d_R]; positions [r]."""
    q_rot = rope_rotate(q_rope_pre, np.asarray(positions, dtype=_F)[:, None], base, layout)
    return np.concatenate([absorb_query(q_nope, w_uk), q_rot], axis=2)


def latent_attention(q_packed, rows_packed, d_latent: int, *, scale: float,
                     heads: Optional[Iterable[int]] = None,
                     rows: Optional[Iterable[int]] = None) -> Dict[str, np.ndarray]:
    """Attention of packed queries [n_q, H, d_c+d_R] over packed rows [n, d_c+d_R].

    The score is one dot product over the concatenated row (content part plus
    position part); the value is the latent part of the same row. Returns
    z [r, h, d_c] and lse [r, h] with the same causal offset as the explicit form.
    """
    qp = np.asarray(q_packed, dtype=_F)
    kv = np.asarray(rows_packed, dtype=_F)
    n, n_q, H = kv.shape[0], qp.shape[0], qp.shape[1]
    rows = np.arange(n_q) if rows is None else np.asarray(list(rows), dtype=np.int64)
    heads = np.arange(H) if heads is None else np.asarray(list(heads), dtype=np.int64)
    vis = visible(n, n_q, rows)
    z = np.zeros((len(rows), len(heads), d_latent), dtype=_F)
    lse = np.zeros((len(rows), len(heads)), dtype=_F)
    for hi, i in enumerate(heads):
        alpha, l = softmax_masked(scale * (qp[rows, i] @ kv.T), vis)
        z[:, hi] = alpha @ kv[:, :d_latent]
        lse[:, hi] = l
    return {"z": z, "lse": lse}


def latent_out_projection(z, w_uv) -> np.ndarray:
    """o[r, i] = W_UV,i z[r, i]: [r, H, d_c] x [H, d_v, d_c] -> [r, H, d_v]."""
    z = np.asarray(z, dtype=_F)
    w_uv = np.asarray(w_uv, dtype=_F)
    out = np.empty((z.shape[0], z.shape[1], w_uv.shape[1]), dtype=_F)
    for i in range(z.shape[1]):
        out[:, i] = z[:, i] @ w_uv[i].T
    return out


# -------------------------------------------------------------- whole layer
def rms_norm(x, weight=None, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps), then times ``weight``.

    The definition is the RMSNorm class of "hands-on DeepSeek MLA" (mean of squares
    over the hidden axis, reciprocal square root with eps, elementwise weight that
    starts at ones); "构建DeepSeek-V3：MLA 架构" step 1 applies it to the compressed
    latent, c_KV = RMSNorm(W_dkv x), and "从零理解 MLA" (engineering notes after the
    decoupled-RoPE check) says the paper adds it after the compressed latent. Here
    everything stays in float64 (the page's class casts to float32 first).
    """
    x = np.asarray(x, dtype=_F)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + _F(eps))
    if weight is not None:
        y = y * np.asarray(weight, dtype=_F)
    return y


def project_inputs(h, weights: Dict[str, np.ndarray], n_heads: int,
                   kv_norm_eps: float = 1e-6) -> Dict[str, np.ndarray]:
    """Projections from hidden states to the attention's inputs.

    c = W_DKV h, k_R(pre-rotation) = W_KR h ("Decoupled RoPE · MLA Part 2", §5 and
    §4.2: the position key comes from h, not from c). When ``weights`` holds
    ``kv_norm_w`` the latent is RMS-normalised with that weight, c = RMSNorm(W_DKV h)
    ("构建DeepSeek-V3：MLA 架构", step 1 and the kv_norm(kv_proj(x)) line of its
    forward pass); without it c is the plain projection, as in the first page's code.
    Content query q_C = W_Q h, or W_UQ W_DQ h with query compression; position query
    from h, or from the compressed query c_Q ("从零理解 MLA", sections "查询压缩" and
    "解耦 RoPE"; "构建DeepSeek-V3：MLA 架构", q_rope = RoPE(W_qr c_Q), with no norm on c_Q).
    """
    h = np.asarray(h, dtype=_F)
    W = {k: np.asarray(v, dtype=_F) for k, v in weights.items()}
    n = h.shape[0]
    c = h @ W["w_dkv"].T
    if "kv_norm_w" in W:
        c = rms_norm(c, W["kv_norm_w"], kv_norm_eps)
    k_rope_pre = h @ W["w_kr"].T
    if "w_q" in W:
        q_c = h @ W["w_q"].T
        q_r = h @ W["w_qr"].T
    else:
        c_q = h @ W["w_dq"].T
        q_c = c_q @ W["w_uq"].T
        q_r = c_q @ W["w_qr"].T
    return {
        "c": c,
        "k_rope_pre": k_rope_pre,
        "q_nope": q_c.reshape(n, n_heads, -1),
        "q_rope_pre": q_r.reshape(n, n_heads, -1),
    }


def full_layer(h, weights: Dict[str, np.ndarray], *, n_heads: int, scale: float, base: float,
               n_q: Optional[int] = None, layout: str = "interleaved",
               keep_scores: bool = False, kv_norm_eps: float = 1e-6) -> Dict[str, np.ndarray]:
    """Whole attention layer from hidden states h [n, d_model].

    The last ``n_q`` tokens (all of them by default, i.e. the square causal mask of a
    full forward) are the query rows; every token is a key.
    """
    p = project_inputs(h, weights, n_heads, kv_norm_eps)
    n = p["c"].shape[0]
    n_q = n if n_q is None else n_q
    res = explicit_attention(p["c"], p["k_rope_pre"], p["q_nope"][n - n_q:], p["q_rope_pre"][n - n_q:],
                             weights["w_uk"], weights["w_uv"], scale=scale, base=base, layout=layout,
                             keep_scores=keep_scores)
    res["u"] = output_projection(res["o"], weights["w_o"])
    res.update(p)
    return res
