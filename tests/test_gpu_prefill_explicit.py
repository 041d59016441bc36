"""GPU parity of the explicit (non-absorbed) prefill, mla_prefill_explicit, through the C ABI:
against the fp64 oracle (whose method is this explicit form) on the same seeded inputs, and,
at the full chunked-prefill size, against the absorbed path's outputs everywhere."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle as O  # noqa: E402
from mla_workloads import CONFIGS, MLAConfig  # noqa: E402

from .gpu_pipeline import assert_close, host_inputs, lib_config, np32, run_pipeline, tdev  # noqa: E402

import mla_decode_decoupled_amd as mla  # noqa: E402


def _run_explicit(hi, run, max_len=None):
    """The explicit prefill over the cache the absorbed pipeline built (same rows, same queries)."""
    cfg = hi.cfg
    lc = lib_config(cfg)
    dt = mla.storage_dtype(lc)
    B, n_q, H = len(hi.lens), cfg.n_q, cfg.n_heads
    max_len = int(hi.lens.max()) if max_len is None else int(max_len)
    ws = torch.empty(mla.mla_prefill_explicit_workspace_size(lc, B, n_q, max_len), dtype=torch.uint8, device="cuda")
    o = torch.full((B, n_q, H, cfg.d_v), float("nan"), dtype=dt, device="cuda")
    lse = torch.full((B, n_q, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_prefill_explicit(lc, tdev(hi.q_nope, dt), tdev(hi.q_rope, dt), run.cache, run.seq_off, run.seq_len,
                             max_len, tdev(hi.w_uk, dt), tdev(hi.w_uv, dt), o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return np32(o), np32(lse)


def _small_cfg(cid, H, n_q, lens):
    base = CONFIGS[1]
    return MLAConfig(cid=cid, name="explicit_small", batch=len(lens), n_heads=H, d_model=base.d_model,
                     q_lora=base.q_lora, d_latent=512, d_rope=64, d_nope=128, d_v=128, n_q=n_q, dtype="bf16",
                     fixed_len=None, ragged_range=(0, 0))


@pytest.mark.parametrize("H,n_q,lens", [
    (4, 40, [100, 57]),          # one ragged query block, two sequences of different lengths
    (8, 300, [300, 333]),        # three query blocks; the first sequence has no cached prefix
    (6, 129, [129 + 31, 1000]),   # 12 (sequence, head) pairs; a query block of one row; a key tail
    (4, 1, [1, 70]),              # one query row (a decode step): a sequence whose only key is itself
], ids=["h4_q40", "h8_q300_empty_prefix", "h6_q129_tail", "h4_q1_single_key"])
def test_explicit_prefill_all_outputs(H, n_q, lens):
    cfg = _small_cfg(200 + H, H, n_q, lens)
    hi = host_inputs(cfg, lens=lens)
    run = run_pipeline(hi)
    o, lse = _run_explicit(hi, run)
    for b in range(len(lens)):
        ref = O.explicit_attention(hi.c[b], hi.k_pre[b], hi.q_nope[b], hi.q_rope[b], hi.w_uk, hi.w_uv,
                                   scale=cfg.softmax_scale, base=cfg.rope_base)
        s1 = assert_close(o[b], ref["o"], "bf16", f"explicit o[{b}]")
        s2 = assert_close(lse[b], ref["lse"], "bf16", f"explicit lse[{b}]")
        # the absorbed path on the same inputs agrees as well
        s3 = assert_close(np32(run.o[b]), ref["o"], "bf16", f"absorbed o[{b}]")
        print(f"H={H} n_q={n_q} seq {b}: explicit o {s1}, lse {s2}; absorbed o {s3}")


@pytest.mark.slow
def test_explicit_prefill_chunked_prefill_workload():
    """The full chunked-prefill workload (2 x 2048 new rows after 2048 cached, 128 heads): sampled
    rows and heads against the oracle, and every output against the absorbed path."""
    cfg = CONFIGS[4]
    hi = host_inputs(cfg)
    run = run_pipeline(hi)
    o, lse = _run_explicit(hi, run)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b, heads, rows in ((1, [0, 127], [0, 1, 1000, 2047]), (0, [64], [2047, 5, 127, 128])):
        ref = O.explicit_attention(hi.c[b], hi.k_pre[b], hi.q_nope[b], hi.q_rope[b], hi.w_uk, hi.w_uv,
                                   scale=cfg.softmax_scale, base=cfg.rope_base, heads=heads, rows=rows)
        assert_close(o[b][rows][:, heads], ref["o"], "bf16", f"sampled o[{b}]")
        assert_close(lse[b][rows][:, heads], ref["lse"], "bf16", f"sampled lse[{b}]")
    # both GPU paths everywhere: each is within the bar of the oracle on the samples, and they
    # compute the same function, so their difference stays within the bar too
    s = assert_close(o, np32(run.o), "bf16", "explicit vs absorbed o (all rows and heads)")
    s2 = assert_close(lse, np32(run.lse), "bf16", "explicit vs absorbed lse (all rows and heads)")
    print("explicit vs absorbed:", s, s2)


def test_explicit_prefill_reference_moves():
    """Scores that climb tile by tile, so that the running reference moves again and again. All
    query rows share one content query; the latent rows of tiles 0-4 are built to score about
    -50, -40, -30, -20 and -10 (natural units) against every head's absorbed query, the later tiles
    are ordinary. Each tile's maximum then exceeds the reference by more than the lazy-rescale
    limit (8 in log2 units), five moves in all, while the outputs and log-sum-exps come from the
    ordinary tiles (the early keys weigh e^-40 and less), so the bf16 bar still applies."""
    from mla_workloads.generate import round_bf16
    lens, n_q, H = [320], 8, 4
    cfg = _small_cfg(210, H, n_q, lens)
    hi = host_inputs(cfg, lens=lens)
    hi.q_nope[0][:] = hi.q_nope[0][0]
    q_abs = O.absorb_query(hi.q_nope[0][:1], hi.w_uk)[0]             # [H, d_c]
    d = sum(q_abs[i] / float(q_abs[i] @ q_abs[i]) for i in range(H))   # q_abs[i] . d ~ 1 for every head
    c = hi.c[0].copy()
    for t in range(5):
        target = -(50.0 - 10.0 * t) / cfg.softmax_scale
        c[32 * t:32 * (t + 1)] = 0.1 * c[32 * t:32 * (t + 1)] + target * d
    hi.c[0] = round_bf16(c)
    run = run_pipeline(hi)
    o, lse = _run_explicit(hi, run)
    ref = O.explicit_attention(hi.c[0], hi.k_pre[0], hi.q_nope[0], hi.q_rope[0], hi.w_uk, hi.w_uv,
                               scale=cfg.softmax_scale, base=cfg.rope_base)
    # the construction holds: each of the first five tiles tops the one before by more than the limit
    s_tile = np.array([[float((q_abs[i] @ hi.c[0][32 * t:32 * (t + 1)].T).max()) for t in range(6)]
                       for i in range(H)]) * cfg.softmax_scale * np.log2(np.e)
    assert np.all(np.diff(s_tile, axis=1) > 8.0), s_tile
    s1 = assert_close(o[0], ref["o"], "bf16", "explicit o")
    s2 = assert_close(lse[0], ref["lse"], "bf16", "explicit lse")
    # the absorbed path on the same inputs: its fixed reference (the first tile's maximum) overflows,
    # and the exact fallback recomputes the chunks
    s3 = assert_close(np32(run.o[0]), ref["o"], "bf16", "absorbed o")
    print(f"tile maxima (log2, content part) {np.round(s_tile[0], 1)}: explicit o {s1}, lse {s2}; absorbed o {s3}")
