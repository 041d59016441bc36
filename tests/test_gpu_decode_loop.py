"""The multi-step decode loop (DecodeStack / DecodeGraph): hidden states go in token by token, the
caches grow, and every layer output matches the oracle's full forward over the whole sequence
with the square causal mask — the check the pages run on their absorbed decode step ("从零理解
MLA", decode loop after the decoupled-RoPE code: step-by-step absorbed outputs equal the naive
forward's rows). The replayed HIP graph is also pinned bit for bit to the same steps launched
eagerly, with eager work and synchronisations between replays."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle as O  # noqa: E402
from mla_workloads import MLAConfig, get_config  # noqa: E402
from mla_workloads import generate as G  # noqa: E402

from .gpu_pipeline import assert_close, lib_config, np32, tdev  # noqa: E402

import mla_decode_decoupled_amd as mla  # noqa: E402
from mla_decode_decoupled_amd.decode_loop import DecodeStack  # noqa: E402

LAYER_KEYS = ("w_dkv", "w_kr", "kv_norm_w", "w_q", "w_dq", "w_uq", "w_qr", "w_uk", "w_uv", "w_o")


def _device_layer(w, dt):
    d = {k: tdev(w[k], dt) for k in LAYER_KEYS if k in w}
    if "w_q" in d:            # no query compression: W_Q takes W_UQ's place
        d["w_uq"] = d.pop("w_q")
    return d


def _oracle_stack(h, layers_host, cfg):
    """Per layer, the full forward of one sequence (square causal mask); returns each layer's u."""
    outs, x = [], h
    for w in layers_host:
        u = O.full_layer(x, w, n_heads=cfg.n_heads, scale=cfg.softmax_scale, base=cfg.rope_base)["u"]
        outs.append(u)
        x = u
    return outs


def test_decode_loop_tiny_two_layers():
    """fp32, 2 layers, 2 sequences of 24 tokens: a 9-token prefill, 5 eager steps, 10 replays."""
    base = get_config(0)
    T, B, P, E = 24, 2, 9, 5
    cfgs = [MLAConfig(cid=110 + l, name="tiny_loop", batch=B, n_heads=base.n_heads, d_model=base.d_model,
                      q_lora=None, d_latent=base.d_latent, d_rope=base.d_rope, d_nope=base.d_nope, d_v=base.d_v,
                      n_q=1, dtype="f32", fixed_len=T, latent_rms_norm=True) for l in range(2)]
    cfg = cfgs[0]
    lc = lib_config(cfg)
    dt = mla.storage_dtype(lc)
    host = [G.full_layer_inputs(c, B * T) for c in cfgs]
    h = host[0]["h"].reshape(B, T, cfg.d_model)
    ref = [_oracle_stack(h[b], host, cfg) for b in range(B)]          # [b][layer] -> [T, d_model]
    layers = [_device_layer(w, dt) for w in host]
    eager = DecodeStack(lc, layers, batch=B, capacity=T + 3)
    graphed = DecodeStack(lc, layers, batch=B, capacity=T + 3)
    hd = tdev(h, dt)

    def check(got, t0, t1, what):
        for b in range(B):
            assert_close(np32(got[b]), ref[b][-1][t0:t1], "f32", f"{what} seq {b} tokens {t0}..{t1 - 1}")

    check(eager.forward(hd[:, :P]), 0, P, "prefill")
    graphed.forward(hd[:, :P])
    for t in range(P, P + E):
        check(eager.forward(hd[:, t:t + 1]), t, t + 1, "eager step")
        graphed.forward(hd[:, t:t + 1])
    g = graphed.capture_decode()
    for t in range(P + E, T):
        want = eager.forward(hd[:, t:t + 1]).clone()
        torch.cuda.synchronize()
        g.h_in.copy_(hd[:, t:t + 1])
        got = g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"replay at token {t} differs from the eager step"
        check(got, t, t + 1, "replayed step")
    assert eager.length == graphed.length == T
    # the rows the two stacks wrote (T per sequence; the rest of each slab is never written) agree
    # bit for bit, and hold the oracle's rows for layer 0
    for l in range(2):
        written_e = eager.caches[l].view(B, T + 3, -1)[:, :T]
        written_g = graphed.caches[l].view(B, T + 3, -1)[:, :T]
        assert torch.equal(written_e, written_g)
    for b in range(B):
        p = O.project_inputs(h[b], {k: host[0][k] for k in LAYER_KEYS if k in host[0]}, cfg.n_heads)
        rows = O.cache_rows(p["c"], p["k_rope_pre"], np.arange(T), cfg.rope_base)
        assert_close(np32(eager.caches[0][b * (T + 3): b * (T + 3) + T]), rows, "f32", f"layer-0 cache seq {b}")


def test_decode_loop_v3_shape_bf16():
    """The DeepSeek-V3 shape, one layer, batch 1: a 64-token prefill (GEMM projections and the
    MFMA attention over 64 query rows), then 4 replayed decode steps (matrix-vector projections,
    head-split attention), against the oracle's forward over all 68 tokens."""
    cfg = get_config(1)
    T, P = 68, 64
    lc = lib_config(cfg)
    dt = mla.storage_dtype(lc)
    w = G.full_layer_inputs(cfg, T)
    ref = O.full_layer(w["h"], w, n_heads=cfg.n_heads, scale=cfg.softmax_scale, base=cfg.rope_base)["u"]
    stack = DecodeStack(lc, [_device_layer(w, dt)], batch=1, capacity=4096)
    hd = tdev(w["h"], dt)[None]
    s = assert_close(np32(stack.forward(hd[:, :P])[0]), ref[:P], "bf16", "prefill u")
    g = stack.capture_decode()
    for t in range(P, T):
        g.h_in.copy_(hd[:, t:t + 1])
        got = np32(g.replay()[0])
        torch.cuda.synchronize()
        s = assert_close(got, ref[t:t + 1], "bf16", f"decode u token {t}")
    print("last step", s)


def test_prefill_route_switch_point():
    """The stack's multi-token step takes the explicit form from the library's switch row count on
    and the absorbed calls just below it; both prefills, and one decode step after each, match the
    oracle's full forward (DeepSeek-V3 shape, one layer, batch 1)."""
    cfg = get_config(1)
    lc = lib_config(cfg)
    dt = mla.storage_dtype(lc)
    switch = next(n for n in range(1, 4097) if mla.mla_prefill_prefers_explicit(lc, 1, n, 4096))
    T = switch + 1
    w = G.full_layer_inputs(cfg, T)
    ref = O.full_layer(w["h"], w, n_heads=cfg.n_heads, scale=cfg.softmax_scale, base=cfg.rope_base)["u"]
    hd = tdev(w["h"], dt)[None]
    for P, path in ((switch, "explicit"), (switch - 1, "absorbed")):
        print(f"prefill of {P} tokens, expecting the {path} form", flush=True)
        stack = DecodeStack(lc, [_device_layer(w, dt)], batch=1, capacity=4096)
        got = np32(stack.forward(hd[:, :P])[0])
        assert stack.last_prefill_path == path
        assert_close(got, ref[:P], "bf16", f"{path} prefill u ({P} tokens)")
        got = np32(stack.forward(hd[:, P:P + 1])[0])
        assert stack.last_prefill_path == "absorbed"
        assert_close(got, ref[P:P + 1], "bf16", f"decode u token {P} after the {path} prefill")
