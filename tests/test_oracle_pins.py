"""Pins for the fp64 oracle: values printed on the pages, closed forms, identities,
library routines and brute force. None of these re-calls the oracle's own
expressions to produce an expected value."""

import json
import math
import os

import numpy as np
import pytest

import oracle as O
from mla_workloads import CONFIGS, MLAConfig
from mla_workloads import generate as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decoupled_rope_hand_example.json")


def _hand():
    with open(GOLDEN) as f:
        g = json.load(f)
    w = {k: np.asarray(v, dtype=np.float64) for k, v in g["constructed"].items()}
    w["w_kr"] = np.asarray(g["w_kr"], dtype=np.float64)
    h = np.asarray(g["h"], dtype=np.float64)
    res = O.full_layer(h, w, n_heads=g["n_heads"], scale=g["scale"], base=10000.0, n_q=1, keep_scores=True)
    return g, res


# ----------------------------------------------------------- hand-worked example
def test_hand_example_position_keys():
    g, res = _hand()
    tol = g["printed_precision"]
    assert np.array_equal(res["k_rope_pre"], np.asarray(g["expected_k_rope_pre"], dtype=float))
    assert np.max(np.abs(res["k_rot"] - np.asarray(g["expected_k_rot"]))) <= tol
    # closed form: [1, 0] turned by p radians is [cos p, sin p] (theta = 1 since d_rope = 2)
    p = np.arange(3.0)
    assert np.max(np.abs(res["k_rot"] - np.stack([np.cos(p), np.sin(p)], 1))) <= 1e-15


def test_hand_example_position_queries():
    g, res = _hand()
    tol = g["printed_precision"]
    assert np.array_equal(res["q_rope_pre"][-1], np.asarray(g["expected_q_rope_pre"], dtype=float))
    assert np.max(np.abs(res["q_rot"][0] - np.asarray(g["expected_q_rot"]))) <= tol


def test_hand_example_scores():
    g, res = _hand()
    tol = g["printed_precision"]
    logits = res["logits"][0]                                   # [heads, keys], scale 1
    assert np.max(np.abs(logits - np.asarray(g["expected_total_scores"]))) <= tol
    pos = np.einsum("hd,jd->hj", res["q_rot"][0], res["k_rot"])
    assert np.max(np.abs(pos - np.asarray(g["expected_position_scores"]))) <= tol
    assert np.max(np.abs((logits - pos) - np.asarray(g["expected_content_scores"]))) <= 1e-15
    # closed forms on the page: head 1 reads cos(s - t), head 2 reads sin(s - t), t = 2
    s = np.arange(3.0)
    assert np.max(np.abs(pos[0] - np.cos(s - 2))) <= 1e-15
    assert np.max(np.abs(pos[1] - np.sin(s - 2))) <= 1e-15


def test_hand_example_shift_invariance():
    """Moving every token 5 positions later leaves the position scores unchanged."""
    g, res = _hand()
    p = O.project_inputs(np.asarray(g["h"], float), {**{k: np.asarray(v, float) for k, v in g["constructed"].items()},
                                                     "w_kr": np.asarray(g["w_kr"], float)}, g["n_heads"])
    a = O.explicit_attention(p["c"], p["k_rope_pre"], p["q_nope"][-1:], p["q_rope_pre"][-1:],
                             np.asarray(g["constructed"]["w_uk"], float), np.asarray(g["constructed"]["w_uv"], float),
                             scale=1.0, base=10000.0, pos_offset=5, keep_scores=True)
    assert np.max(np.abs(a["logits"] - res["logits"])) <= 1e-14


def test_cache_element_counts():
    with open(GOLDEN) as f:
        g = json.load(f)
    for d_c, d_r, total in g["expected_cache_elements"].values():
        assert d_c + d_r == total
    assert CONFIGS[1].row == 576
    assert MLAConfig(cid=99, name="p3toy", batch=1, n_heads=4, d_model=128, q_lora=48, d_latent=32, d_rope=8,
                     d_nope=16, d_v=16, n_q=1, dtype="f32", fixed_len=10).row == 40


# ------------------------------------------------------------------- RoPE pins
def test_rope_relative_identity():
    """(R_t q)^T (R_s k) = q^T R_(s-t) k for random vectors and positions."""
    rng = np.random.default_rng(7)
    for d in (2, 8, 64):
        for _ in range(20):
            q, k = rng.standard_normal(d), rng.standard_normal(d)
            t, s = rng.integers(0, 200000, size=2)
            lhs = O.rope_rotate(q, t, 10000.0) @ O.rope_rotate(k, s, 10000.0)
            rhs = q @ O.rope_rotate(k, s - t, 10000.0)
            assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs))


def test_rope_norm_preserved_and_zero_position_identity():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 64))
    assert np.array_equal(O.rope_rotate(x, np.zeros(5), 10000.0), x)
    y = O.rope_rotate(x, np.arange(5) * 1000.0, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), atol=1e-12)


def _hf_rope(d, base, pos, x64):
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers")
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    from transformers.models.deepseek_v3.modeling_deepseek_v3 import apply_rotary_pos_emb_interleave

    cfg = LlamaConfig(hidden_size=4 * d, num_attention_heads=4, head_dim=d, rope_theta=base)
    emb = LlamaRotaryEmbedding(cfg).double()
    x = torch.from_numpy(x64)[None, None]
    cos, sin = emb(x, torch.from_numpy(pos)[None])
    half, _ = apply_rotary_pos_emb(x, x, cos, sin)
    inter, _ = apply_rotary_pos_emb_interleave(x, x, cos, sin)
    return half[0, 0].numpy(), inter[0, 0].numpy()


@pytest.mark.parametrize("d", [8, 64])
def test_rope_matches_library_routines(d):
    """Both pairings against the transformers RoPE routines (frequencies base^(-2j/d)).

    The library's interleaved routine returns its result de-interleaved
    (evens then odds), so the oracle's interleaved output is compared after that
    permutation. The library computes its inverse frequencies in float32, so the
    angles may differ by a few float32 ulps of theta_j times the position.
    """
    rng = np.random.default_rng(d)
    pos = rng.integers(0, 300, size=12)
    x = rng.standard_normal((12, d))
    half, inter = _hf_rope(d, 10000.0, pos, x)
    tol = 8 * 2.0 ** -24 * pos.max() * 2 * np.abs(x).max()
    assert np.max(np.abs(O.rope_rotate(x, pos, 10000.0, "half") - half)) <= tol
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    assert np.max(np.abs(O.rope_rotate(x, pos, 10000.0, "interleaved")[:, perm] - inter)) <= tol


def test_half_split_is_permuted_interleaved():
    rng = np.random.default_rng(3)
    d = 16
    x = rng.standard_normal((6, d))
    pos = rng.integers(0, 5000, size=6)
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])   # interleaved index -> half index
    a = O.rope_rotate(x[:, perm], pos, 10000.0, "half")
    b = O.rope_rotate(x, pos, 10000.0, "interleaved")[:, perm]
    assert np.max(np.abs(a - b)) <= 1e-13


# ---------------------------------------------------- attention: library routine
def _random_case(rng, H=3, n=11, n_q=4, d_c=6, d_nope=4, d_r=4, d_v=5):
    return dict(
        c=rng.standard_normal((n, d_c)), k_rope_pre=rng.standard_normal((n, d_r)),
        q_nope=rng.standard_normal((n_q, H, d_nope)), q_rope_pre=rng.standard_normal((n_q, H, d_r)),
        w_uk=rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c),
    )


@pytest.mark.parametrize("d_r", [0, 4])
def test_explicit_attention_matches_torch_sdpa(d_r):
    """Scaled, offset-causal attention against torch's scaled_dot_product_attention (fp64, CPU).

    Keys and values are rebuilt with torch.nn.functional.linear, the nn.Linear
    ([out, in]) convention the pages use for W_UK / W_UV. d_r = 0 is the MLA
    without a position channel.
    """
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(11 + d_r)
    cs = _random_case(rng, d_r=d_r)
    H, n_q = cs["q_nope"].shape[1], cs["q_nope"].shape[0]
    n = cs["c"].shape[0]
    scale = 1.0 / math.sqrt(4 + d_r)
    res = O.explicit_attention(**cs, scale=scale, base=10000.0)
    c = torch.from_numpy(cs["c"])
    k_rot = torch.from_numpy(res["k_rot"])
    mask = torch.ones(n_q, n, dtype=torch.bool).tril(diagonal=n - n_q)
    for i in range(H):
        k = torch.cat([F.linear(c, torch.from_numpy(cs["w_uk"][i])), k_rot], dim=1)
        v = F.linear(c, torch.from_numpy(cs["w_uv"][i]))
        q = torch.cat([torch.from_numpy(cs["q_nope"][:, i]), torch.from_numpy(res["q_rot"][:, i])], dim=1)
        ref = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask, scale=scale)[0]
        assert np.max(np.abs(res["o"][:, i] - ref.numpy())) <= 1e-12
        lse_ref = torch.logsumexp((q @ k.T * scale).masked_fill(~mask, -math.inf), dim=-1)
        assert np.max(np.abs(res["lse"][:, i] - lse_ref.numpy())) <= 1e-12


def test_brute_force_tiny():
    """Pure-Python loops (math.cos/sin/exp, no numpy algebra) on a tiny case."""
    rng = np.random.default_rng(5)
    H, n, n_q, d_c, d_nope, d_r, d_v = 2, 5, 2, 3, 2, 4, 2
    cs = _random_case(rng, H=H, n=n, n_q=n_q, d_c=d_c, d_nope=d_nope, d_r=d_r, d_v=d_v)
    base, scale = 100.0, 0.37
    res = O.explicit_attention(**cs, scale=scale, base=base)

    def rot(vec, p):
        out = list(vec)
        for j in range(len(vec) // 2):
            ang = p * base ** (-2.0 * j / len(vec))
            a, b = vec[2 * j], vec[2 * j + 1]
            out[2 * j] = a * math.cos(ang) - b * math.sin(ang)
            out[2 * j + 1] = a * math.sin(ang) + b * math.cos(ang)
        return out

    C = cs["c"].tolist()
    kr = [rot(cs["k_rope_pre"][j].tolist(), j) for j in range(n)]
    for t in range(n_q):
        pos = n - n_q + t
        for i in range(H):
            W = cs["w_uk"][i].tolist()
            Wv = cs["w_uv"][i].tolist()
            qn = cs["q_nope"][t, i].tolist()
            qr = rot(cs["q_rope_pre"][t, i].tolist(), pos)
            scores = []
            for j in range(pos + 1):
                kc = [sum(W[a][cc] * C[j][cc] for cc in range(d_c)) for a in range(d_nope)]
                dot = sum(qn[a] * kc[a] for a in range(d_nope)) + sum(qr[r] * kr[j][r] for r in range(d_r))
                scores.append(scale * dot)
            mx = max(scores)
            ex = [math.exp(s - mx) for s in scores]
            tot = sum(ex)
            for vv in range(d_v):
                o = sum(ex[j] / tot * sum(Wv[vv][cc] * C[j][cc] for cc in range(d_c)) for j in range(pos + 1))
                assert abs(o - res["o"][t, i, vv]) <= 1e-12
            for cc in range(d_c):
                zz = sum(ex[j] / tot * C[j][cc] for j in range(pos + 1))
                assert abs(zz - res["z"][t, i, cc]) <= 1e-12
            assert abs(mx + math.log(tot) - res["lse"][t, i]) <= 1e-12


# ------------------------------------------------------------ closed forms
def test_two_key_logistic_closed_form():
    """Two keys with content logits a, b (no position signal): alpha_0 = 1/(1 + e^{scale (b - a)})."""
    a, b = 0.7, -1.9
    c = np.array([[1.0, 0.0], [0.0, 1.0]])
    w_uk = np.eye(2)[None]
    res = O.explicit_attention(c, np.zeros((2, 2)), np.array([[[a, b]]]), np.zeros((1, 1, 2)),
                               w_uk, w_uk, scale=0.5, base=10000.0, keep_scores=True)
    assert abs(res["alpha"][0, 0, 0] - 1.0 / (1.0 + math.exp(0.5 * (b - a)))) <= 1e-15
    assert abs(res["lse"][0, 0] - math.log(math.exp(0.5 * a) + math.exp(0.5 * b))) <= 1e-14


def test_single_key_returns_its_latent():
    rng = np.random.default_rng(2)
    cs = _random_case(rng, n=1, n_q=1)
    res = O.explicit_attention(**cs, scale=0.3, base=10000.0)
    for i in range(cs["w_uk"].shape[0]):
        assert np.array_equal(res["z"][0, i], cs["c"][0])
        # o = W_UV,i c_0 with W_UV,i stored [d_v, d_c]
        assert np.allclose(res["o"][0, i], [sum(cs["w_uv"][i, v, k] * cs["c"][0, k] for k in range(6))
                                            for v in range(cs["w_uv"].shape[1])], atol=1e-14)


def test_zero_queries_give_uniform_weights():
    rng = np.random.default_rng(4)
    cs = _random_case(rng, n=9, n_q=3)
    cs["q_nope"][:] = 0
    cs["q_rope_pre"][:] = 0
    res = O.explicit_attention(**cs, scale=0.3, base=10000.0, keep_scores=True)
    for t in range(3):
        nv = 9 - 3 + t + 1
        assert np.allclose(res["alpha"][t, :, :nv], 1.0 / nv, atol=1e-15)
        assert np.all(res["alpha"][t, :, nv:] == 0)
        assert np.allclose(res["z"][t], cs["c"][:nv].mean(axis=0)[None], atol=1e-14)
        assert np.allclose(res["lse"][t], math.log(nv), atol=1e-14)


def test_softmax_rows_sum_to_one_and_respect_mask():
    rng = np.random.default_rng(6)
    cs = _random_case(rng, n=20, n_q=5)
    res = O.explicit_attention(**cs, scale=0.4, base=10000.0, keep_scores=True)
    assert np.allclose(res["alpha"].sum(-1), 1.0, atol=1e-12)
    vis = O.visible(20, 5)
    assert np.all(res["alpha"][~np.broadcast_to(vis[:, None], res["alpha"].shape)] == 0)


def test_identical_heads_identical_outputs():
    rng = np.random.default_rng(9)
    cs = _random_case(rng, H=3)
    for k in ("q_nope", "q_rope_pre"):
        cs[k][:, 1:] = cs[k][:, :1]
    for k in ("w_uk", "w_uv"):
        cs[k][1:] = cs[k][:1]
    res = O.explicit_attention(**cs, scale=0.4, base=10000.0)
    assert np.array_equal(res["o"][:, 1], res["o"][:, 0]) and np.array_equal(res["o"][:, 2], res["o"][:, 0])


def test_prefill_row_equals_truncated_decode():
    """Row t of a multi-row call equals one decode step over the first n - n_q + t + 1 keys."""
    rng = np.random.default_rng(10)
    cs = _random_case(rng, n=14, n_q=5)
    full = O.explicit_attention(**cs, scale=0.4, base=10000.0)
    for t in range(5):
        m = 14 - 5 + t + 1
        one = O.explicit_attention(cs["c"][:m], cs["k_rope_pre"][:m], cs["q_nope"][t:t + 1],
                                   cs["q_rope_pre"][t:t + 1], cs["w_uk"], cs["w_uv"], scale=0.4, base=10000.0)
        assert np.max(np.abs(one["o"][0] - full["o"][t])) <= 1e-13
        assert np.max(np.abs(one["z"][0] - full["z"][t])) <= 1e-13


def test_sampled_heads_and_rows_match_full():
    rng = np.random.default_rng(12)
    cs = _random_case(rng, H=5, n=13, n_q=4)
    full = O.explicit_attention(**cs, scale=0.4, base=10000.0)
    part = O.explicit_attention(**cs, scale=0.4, base=10000.0, heads=[4, 1], rows=[3, 0])
    assert np.array_equal(part["o"], full["o"][[3, 0]][:, [4, 1]])
    assert np.array_equal(part["lse"], full["lse"][[3, 0]][:, [4, 1]])


# ----------------------------------------------------- absorbed == explicit
TOY_SHAPES = [
    # the first page's toy: d_model 64, 4 heads, d_c 8, d_rope 4, 10 tokens (d_h = 16)
    dict(H=4, d_model=64, d_c=8, d_r=4, d_h=16, q_lora=None, n=10),
    # the third page's toy: d 128, 4 heads, d_head 16, d_c 32, d_cq 48, d_rope 8, 10 tokens
    dict(H=4, d_model=128, d_c=32, d_r=8, d_h=16, q_lora=48, n=10),
    # the tiny fp32 workload's shapes
    dict(H=4, d_model=64, d_c=32, d_r=8, d_h=16, q_lora=None, n=129),
]


@pytest.mark.parametrize("shape", TOY_SHAPES, ids=["toy_p1", "toy_p3", "tiny"])
def test_absorbed_equals_explicit(shape):
    cfg = MLAConfig(cid=50 + shape["d_c"], name="toy", batch=1, n_heads=shape["H"], d_model=shape["d_model"],
                    q_lora=shape["q_lora"], d_latent=shape["d_c"], d_rope=shape["d_r"], d_nope=shape["d_h"],
                    d_v=shape["d_h"], n_q=shape["n"], dtype="f32", fixed_len=shape["n"], latent_rms_norm=False)
    w = G.full_layer_inputs(cfg, shape["n"])
    full = O.full_layer(w["h"], w, n_heads=cfg.n_heads, scale=cfg.softmax_scale, base=cfg.rope_base)
    n = shape["n"]
    rows = O.cache_rows(full["c"], full["k_rope_pre"], np.arange(n), cfg.rope_base)
    qp = O.packed_query(full["q_nope"], full["q_rope_pre"], np.arange(n), w["w_uk"], cfg.rope_base)
    lat = O.latent_attention(qp, rows, cfg.d_latent, scale=cfg.softmax_scale)
    assert np.max(np.abs(lat["z"] - full["z"])) <= 1e-10
    assert np.max(np.abs(lat["lse"] - full["lse"])) <= 1e-10
    o_abs = O.latent_out_projection(lat["z"], w["w_uv"])
    assert np.max(np.abs(o_abs - full["o"])) <= 1e-10
    # token-by-token decode with a growing cache reproduces the full forward (append, then attend)
    for t in (0, n // 2, n - 1):
        step = O.latent_attention(qp[t:t + 1], rows[:t + 1], cfg.d_latent, scale=cfg.softmax_scale)
        assert np.max(np.abs(O.latent_out_projection(step["z"], w["w_uv"]) - full["o"][t:t + 1])) <= 1e-10


def test_query_compression_path_uses_library_linear():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg = MLAConfig(cid=77, name="toy", batch=1, n_heads=4, d_model=128, q_lora=48, d_latent=32, d_rope=8,
                    d_nope=16, d_v=16, n_q=10, dtype="f32", fixed_len=10, latent_rms_norm=False)
    w = G.full_layer_inputs(cfg, 10)
    p = O.project_inputs(w["h"], w, 4)
    T = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in w.items()}
    cq = F.linear(T["h"], T["w_dq"])
    assert np.allclose(p["q_nope"].reshape(10, -1), F.linear(cq, T["w_uq"]).numpy(), atol=1e-12)
    assert np.allclose(p["q_rope_pre"].reshape(10, -1), F.linear(cq, T["w_qr"]).numpy(), atol=1e-12)
    assert np.allclose(p["c"], F.linear(T["h"], T["w_dkv"]).numpy(), atol=1e-12)
    assert np.allclose(p["k_rope_pre"], F.linear(T["h"], T["w_kr"]).numpy(), atol=1e-12)


def test_output_projection_concatenates_heads_in_order():
    """u = W_O concat_i(o_i) with a head-major concatenation ("Decoupled RoPE · MLA Part 2", §5
    step 5): W_O made of one-hot rows picks single entries o[i, v] (a transposed W_O or a
    v-major concatenation would pick others), and W_O = [I I ... I], one identity block per head,
    sums the heads' outputs."""
    rng = np.random.default_rng(7)
    R, H, dv = 3, 4, 5
    o = rng.standard_normal((R, H, dv))
    picks = [(0, 0), (3, 4), (1, 2), (2, 0), (3, 1), (0, 4)]
    w_sel = np.zeros((len(picks), H * dv))
    for n, (i, v) in enumerate(picks):
        w_sel[n, i * dv + v] = 1.0
    u = O.output_projection(o, w_sel)
    assert u.shape == (R, len(picks))
    for n, (i, v) in enumerate(picks):
        assert np.array_equal(u[:, n], o[:, i, v])
    w_sum = np.tile(np.eye(dv), (1, H))
    assert np.max(np.abs(O.output_projection(o, w_sum) - o.sum(axis=1))) <= 1e-15


# ------------------------------------------------------------- latent RMSNorm
def test_rms_norm_matches_library_routine():
    """RMSNorm as defined by the RMSNorm class of "hands-on DeepSeek MLA" is the routine torch
    ships as torch.nn.functional.rms_norm (float64 here, no float32 cast)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 32)) * 3.0
    w = 1.0 + 0.25 * rng.standard_normal(32)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (32,), torch.from_numpy(w), 1e-6).numpy()
    assert np.max(np.abs(O.rms_norm(x, w, 1e-6) - ref)) <= 1e-12


def test_rms_norm_closed_forms():
    eps = 1e-6
    w = np.arange(1.0, 9.0)
    # a constant vector a*1 has RMS |a|: every entry becomes a / sqrt(a^2 + eps), times the gain
    for a in (2.5, -0.75):
        y = O.rms_norm(np.full(8, a), w, eps)
        assert np.max(np.abs(y - w * a / math.sqrt(a * a + eps))) <= 1e-15
    # [3, 4]: mean of squares 12.5
    assert np.max(np.abs(O.rms_norm(np.array([3.0, 4.0]), None, 0.0) - np.array([3.0, 4.0]) / math.sqrt(12.5))) <= 1e-15
    # eps = 0 and a unit gain: RMS exactly 1 per row, and a positive rescaling of the input changes nothing
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 64))
    y = O.rms_norm(x, None, 0.0)
    assert np.max(np.abs(np.sqrt(np.mean(y * y, axis=-1)) - 1.0)) <= 1e-14
    assert np.max(np.abs(O.rms_norm(7.0 * x, None, 0.0) - y)) <= 1e-14


def test_normalised_latent_projection_uses_library_routines():
    """c = RMSNorm(W_DKV h) ("构建DeepSeek-V3：MLA 架构", step 1) when the weights carry the
    latent's norm gain; the position key and the queries are not normalised."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg = MLAConfig(cid=78, name="toy", batch=1, n_heads=4, d_model=128, q_lora=48, d_latent=32, d_rope=8,
                    d_nope=16, d_v=16, n_q=6, dtype="f32", fixed_len=6, latent_rms_norm=True)
    w = G.full_layer_inputs(cfg, 6)
    assert "kv_norm_w" in w and np.std(w["kv_norm_w"]) > 0.1
    p = O.project_inputs(w["h"], w, 4, kv_norm_eps=1e-6)
    T = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in w.items()}
    c_ref = F.rms_norm(F.linear(T["h"], T["w_dkv"]), (32,), T["kv_norm_w"], 1e-6).numpy()
    assert np.max(np.abs(p["c"] - c_ref)) <= 1e-12
    assert np.allclose(p["k_rope_pre"], F.linear(T["h"], T["w_kr"]).numpy(), atol=1e-12)
    cq = F.linear(T["h"], T["w_dq"])
    assert np.allclose(p["q_nope"].reshape(6, -1), F.linear(cq, T["w_uq"]).numpy(), atol=1e-12)
    # the whole layer uses the normalised latent for keys, values and the cache
    full = O.full_layer(w["h"], w, n_heads=4, scale=cfg.softmax_scale, base=cfg.rope_base)
    assert np.max(np.abs(full["c"] - c_ref)) <= 1e-12
