"""GPU parity: the HIP path through the C ABI against the fp64 oracle, on the same seeded inputs.

Bar (per output): fp32 storage -> max|err| <= 1e-5; bf16 storage -> max|err| <= 2e-2 and
rel-L2 <= 1e-2. Cache latents are copies and must match bit for bit; rotated position keys
must sit within one bf16 rounding (2^-8 relative) or float32 rounding of the fp64 value.
"""

import json
import math
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_decode_decoupled_amd as mla  # noqa: E402
import oracle as O  # noqa: E402
from mla_workloads import CONFIGS, MLAConfig  # noqa: E402
from mla_workloads import generate as G  # noqa: E402

from .gpu_pipeline import assert_close, host_inputs, lib_config, np32, run_pipeline, tdev  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _oracle(hi, b, heads=None, rows=None, scale=None):
    cfg = hi.cfg
    return O.explicit_attention(hi.c[b], hi.k_pre[b], hi.q_nope[b], hi.q_rope[b], hi.w_uk, hi.w_uv,
                                scale=cfg.softmax_scale if scale is None else scale, base=cfg.rope_base,
                                heads=heads, rows=rows)


def _check_cache(run, hi, b):
    cfg = hi.cfg
    n = int(hi.lens[b])
    off = int(run.seq_off[b].item())
    rows = np32(run.cache[off:off + n])
    assert np.array_equal(rows[:, :cfg.d_latent], hi.c[b].astype(np.float64)), "latent rows must be exact copies"
    k_ref = O.rope_rotate(hi.k_pre[b], np.arange(n), cfg.rope_base)
    rel = 2.0 ** -8 if cfg.dtype == "bf16" else 2.0 ** -23
    err = np.abs(rows[:, cfg.d_latent:] - k_ref)
    assert np.all(err <= rel * np.abs(k_ref) + 1e-7), f"rotated keys: max err {err.max():.3e}"


def _check_qpacked(run, hi, b, rows=None):
    cfg = hi.cfg
    n = int(hi.lens[b])
    rows = np.arange(cfg.n_q) if rows is None else np.asarray(rows)
    pos = n - cfg.n_q + rows
    ref = O.packed_query(hi.q_nope[b][rows], hi.q_rope[b][rows], pos, hi.w_uk, cfg.rope_base)
    assert_close(np32(run.q_packed[b][rows]), ref, cfg.dtype, f"q_packed[{b}]")


def _check_outputs(run, hi, b, heads=None, rows=None, scale=None):
    cfg = hi.cfg
    ref = _oracle(hi, b, heads=heads, rows=rows, scale=scale)
    sel_r = np.arange(cfg.n_q) if rows is None else np.asarray(rows)
    sel_h = np.arange(cfg.n_heads) if heads is None else np.asarray(heads)
    z = np32(run.z[b])[sel_r][:, sel_h]
    lse = np32(run.lse[b])[sel_r][:, sel_h]
    o = np32(run.o[b])[sel_r][:, sel_h]
    stats = {
        "z": assert_close(z, ref["z"], cfg.dtype, f"z[{b}]"),
        "lse": assert_close(lse, ref["lse"], cfg.dtype, f"lse[{b}]"),
        "o": assert_close(o, ref["o"], cfg.dtype, f"o[{b}]"),
    }
    print(f"seq {b}: " + ", ".join(f"{k} max {v['max_err']:.2e} relL2 {v['rel_l2']:.2e}" for k, v in stats.items()),
          flush=True)
    return stats


# ------------------------------------------------------------------ the five workloads
def test_tiny_fp32_all_outputs():
    hi = host_inputs(CONFIGS[0])
    run = run_pipeline(hi)
    _check_cache(run, hi, 0)
    _check_qpacked(run, hi, 0)
    _check_outputs(run, hi, 0)


def test_v3_decode_4k_all_heads():
    hi = host_inputs(CONFIGS[1])
    run = run_pipeline(hi)
    _check_cache(run, hi, 0)
    _check_qpacked(run, hi, 0)
    _check_outputs(run, hi, 0)


@pytest.mark.parametrize("cid,n_splits", [(0, 1), (0, 7), (0, 256), (1, 0), (1, 1), (1, 3), (1, 64), (1, 256)])
def test_split_count_does_not_change_results(cid, n_splits):
    """fp32: only the float32 summation order changes -> 1e-5. n_splits = 0 on the batch-1 4K
    workload is the library's own choice: the head-split kernel, whose scores are summed from four
    partial dot products.

    bf16: each chunk rounds its probabilities to bf16 relative to its own reference max, so the
    rounding (at most 2^-9 relative per weight, independent across keys) differs between split
    counts; the latent sum inherits ~1e-3 relative noise. Bound: rel-L2 <= 5e-3, max <= 2e-3.
    The log-sum-exp is accumulated in float32 either way -> 1e-5.
    """
    hi = host_inputs(CONFIGS[cid])
    base = run_pipeline(hi, n_splits=9)
    other = run_pipeline(hi, n_splits=n_splits)
    zb, zo = np32(base.z), np32(other.z)
    dz = np.abs(zo - zb).max()
    rel = np.linalg.norm(zo - zb) / np.linalg.norm(zb)
    dl = np.abs(np32(other.lse) - np32(base.lse)).max()
    print(f"split {n_splits} vs 9: max|dz| {dz:.2e} rel-L2 {rel:.2e} max|dlse| {dl:.2e}", flush=True)
    assert dl <= 1e-5
    if CONFIGS[cid].dtype == "f32":
        assert dz <= 1e-5
    else:
        assert dz <= 2e-3 and rel <= 5e-3


@pytest.mark.parametrize("n_splits", [2, 3])
def test_fast_kernel_chunk_tails(n_splits):
    """The 128-head MFMA kernel with a caller's split count (chunks of ceil(100 / n_splits) keys) on
    lengths whose chunks end in every way a chunk can: a partial last tile of a chunk of two tiles,
    which moves back to end at the chunk's last key and masks the rows it repeats (33 keys: a
    31-row repeat); a chunk shorter than one tile, whose one tile re-reads its last key; exact tiles.
    All heads and outputs against the oracle."""
    lens = [100, 90, 33, 64, 65]
    cfg = MLAConfig(**{**CONFIGS[1].__dict__, "batch": len(lens)})
    hi = host_inputs(cfg, lens=lens)
    run = run_pipeline(hi, n_splits=n_splits)
    for b in range(len(lens)):
        _check_outputs(run, hi, b)


def test_fast_kernel_causal_rows_with_fixed_splits():
    """Several causal query rows per sequence with a caller's split count on the 128-head kernel:
    40 new rows on 300 and 137 keys in chunks of 100 keys, so every row of the first sequence has
    three chunks (the last one ending in a partial tile), while the rows of the second see 98 to 137
    keys: its first rows fit one chunk (z written directly, their second chunk has no keys and does
    nothing) and its later rows take two (partials and the merge). All rows and heads against the
    oracle."""
    lens = [300, 137]
    cfg = MLAConfig(**{**CONFIGS[1].__dict__, "cid": 260, "batch": len(lens), "n_q": 40})
    hi = host_inputs(cfg, lens=lens)
    run = run_pipeline(hi, n_splits=3)
    for b in range(len(lens)):
        _check_outputs(run, hi, b)


def test_ragged_batch_sampled():
    cfg = CONFIGS[2]
    hi = host_inputs(cfg)
    run = run_pipeline(hi, n_splits=4)
    lens = hi.lens
    picks = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 17})
    heads = [0, 63, 127]
    for b in picks:
        _check_cache(run, hi, b)
        _check_qpacked(run, hi, b)
        _check_outputs(run, hi, b, heads=heads)
    # a sequence attended alone (same chunking, same packed queries) equals the same sequence
    # inside the batch, bit for bit: no other sequence leaks into its result. (The projections
    # take a different path for 1 row than for 64, so the packed queries are passed over.)
    b = picks[-1]
    alone = host_inputs(MLAConfig(**{**cfg.__dict__, "batch": 1}), lens=[int(lens[b])])
    alone.c, alone.k_pre = [hi.c[b]], [hi.k_pre[b]]
    alone.q_nope, alone.q_rope = hi.q_nope[b:b + 1], hi.q_rope[b:b + 1]
    run1 = run_pipeline(alone, n_splits=4, max_len=int(lens.max()))
    lc = lib_config(cfg)
    max_len = int(lens.max())
    z1 = torch.empty_like(run1.z)
    lse1 = torch.empty_like(run1.lse)
    ws = torch.empty(max(mla.mla_decode_attn_workspace_size(lc, 1, 1, max_len, 4), 1), dtype=torch.uint8,
                     device="cuda")
    mla.mla_decode_attn(lc, run.q_packed[b:b + 1].contiguous(), run1.cache, run1.seq_off, run1.seq_len, max_len,
                        z1, lse1, n_splits=4, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(np32(z1[0]), np32(run.z[b]))
    assert np.array_equal(np32(lse1[0]), np32(run.lse[b]))


def test_head_split_small_batch_mixed_lengths():
    """Few query rows over short histories take the head-split kernel (four workgroups per chunk,
    one per block of 32 heads, the waves splitting the dims and the latent columns). The lengths
    give a row short enough for a single chunk (written directly), rows cut into several chunks
    (merged) and tail tiles; two queries per sequence give rows of different visible length.
    Heads from all four blocks, at both ends of each block."""
    cfg = MLAConfig(**{**CONFIGS[1].__dict__, "batch": 3, "n_q": 2})
    hi = host_inputs(cfg, lens=[41, 700, 3001])
    run = run_pipeline(hi)
    for b in range(3):
        _check_cache(run, hi, b)
        _check_qpacked(run, hi, b)
        _check_outputs(run, hi, b, heads=[0, 31, 32, 63, 64, 95, 96, 127])


def test_ragged_batch_balanced_chunks():
    """The library's own chunking of a ragged batch (every row cut into chunks of one common
    length, sized so that the whole batch fills one grid): the shortest, the longest and two
    middle sequences against the oracle."""
    cfg = CONFIGS[2]
    hi = host_inputs(cfg)
    run = run_pipeline(hi)
    lens = hi.lens
    for b in sorted({int(np.argmin(lens)), int(np.argmax(lens)), 5, 40}):
        # both ends of every 32-head block: wave w of the attention kernel owns heads 32w .. 32w + 31
        _check_outputs(run, hi, b, heads=[0, 31, 32, 63, 64, 95, 96, 127])


def test_ragged_batch_plan_extremes():
    """The balanced chunk plan on an extreme length mix: 40 rows, among them single-key rows, rows one
    key either side of a tile boundary and rows of 4097, 12345 and 20000 keys, so that the bisected
    chunk bound cuts the long rows into many evenly split chunks while short rows take one (a row
    whose keys all fit one chunk writes z directly). Every row against the oracle, at both ends of
    every 32-head block."""
    cfg = CONFIGS[2]
    lens = [1, 2, 31, 32, 33, 63, 64, 65, 20000, 1, 96, 97, 12345, 1, 5, 4097, 128, 129, 1, 3,
            200, 33, 1, 700, 31, 1000, 1, 2, 64, 65, 160, 1, 4, 999, 1, 300, 32, 1, 77, 2048]
    hi = host_inputs(cfg, lens=lens)
    run = run_pipeline(hi)
    for b in range(len(lens)):
        _check_outputs(run, hi, b, heads=[0, 31, 32, 63, 64, 95, 96, 127])


@pytest.mark.slow
def test_long_context_128k_sampled():
    cfg = CONFIGS[3]
    hi = host_inputs(cfg)
    run = run_pipeline(hi, n_splits=cfg.n_splits)
    _check_cache(run, hi, 0)
    _check_qpacked(run, hi, 3)
    # both ends of every 32-head block (wave w of the attention kernel owns heads 32w .. 32w + 31)
    _check_outputs(run, hi, 0, heads=[0, 31, 32, 63, 64, 95, 96, 127])
    _check_outputs(run, hi, 3, heads=[5, 64, 100])


@pytest.mark.slow
def test_chunked_prefill_sampled():
    cfg = CONFIGS[4]
    hi = host_inputs(cfg)
    run = run_pipeline(hi)
    _check_cache(run, hi, 1)
    _check_qpacked(run, hi, 1, rows=[0, 1, 1000, 2047])
    # both ends of every 32-head block: wave w of the attention kernel scores heads 32w .. 32w + 31,
    # and every wave writes its 128 latent columns of all heads' z
    _check_outputs(run, hi, 1, heads=[0, 31, 32, 63, 64, 95, 96, 127], rows=[0, 1, 1000, 2047])
    _check_outputs(run, hi, 0, heads=[64], rows=[2047, 5])


@pytest.mark.parametrize("n_q", [15, 16, 100])
def test_projection_row_counts(n_q):
    """DeepSeek shape with a few query rows: 15 rows take the matrix-vector projections, 16 and
    100 the MFMA GEMMs (100 leaves a partial 64-row tile). Every row and head of q_packed and o,
    and z of every row for a subset of heads, against the oracle."""
    cfg = MLAConfig(**{**CONFIGS[1].__dict__, "cid": 210 + n_q, "n_q": n_q, "fixed_len": n_q + 200})
    hi = host_inputs(cfg)
    run = run_pipeline(hi)
    _check_qpacked(run, hi, 0)
    _check_outputs(run, hi, 0, heads=[0, 31, 64, 127])
    # o for every head: the projection of the GPU's own z (isolates the output projection)
    z = np32(run.z[0])
    o_ref = O.latent_out_projection(z, hi.w_uv)
    assert_close(np32(run.o[0]), o_ref, cfg.dtype, "o from GPU z")


@pytest.mark.parametrize("dtype,n_rows,d_model", [("f32", 3, 64), ("bf16", 1, 200), ("bf16", 3, 7168),
                                                  ("bf16", 40, 300)])
def test_w_o_projection(dtype, n_rows, d_model):
    """The optional layer output u = W_O concat_i(o_i) of mla_out_proj, every element against the
    oracle's output projection of its fp64 o. fp32 (4 heads, d_v 16) takes the generic kernel;
    the bf16 DeepSeek shape (K = 128 x 128) takes the matrix-vector kernel for 1 and 3 rows (200
    outputs leave a partial block) and the MFMA GEMM for 40 rows (partial tiles both ways)."""
    if dtype == "f32":
        cfg = _small_cfg(220, "f32")
    else:
        cfg = MLAConfig(**{**CONFIGS[1].__dict__, "cid": 221})
    H, dv, dc = cfg.n_heads, cfg.d_v, cfg.d_latent
    rng = np.random.default_rng(1000 + n_rows)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16

    def stored(x):   # the values the GPU sees, back on the host in float64
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(tdt)
        return t, t.to(torch.float64).numpy()

    z = rng.standard_normal((n_rows, H, dc)).astype(np.float32)
    w_uv_t, w_uv = stored(rng.standard_normal((H, dv, dc)) / np.sqrt(dc))
    w_o_t, w_o = stored(rng.standard_normal((d_model, H * dv)) / np.sqrt(H * dv))
    lc = lib_config(cfg)
    o = torch.empty((n_rows, H, dv), dtype=tdt, device="cuda")
    u = torch.empty((n_rows, d_model), dtype=tdt, device="cuda")
    mla.mla_out_proj(lc, torch.from_numpy(z).cuda(), w_uv_t.cuda(), o, w_o_t.cuda(), u)
    torch.cuda.synchronize()
    o_ref = O.latent_out_projection(z, w_uv)
    u_ref = O.output_projection(o_ref, w_o)
    assert_close(np32(o), o_ref, cfg.dtype, "o")
    st = assert_close(np32(u), u_ref, cfg.dtype, "u")
    print(f"u: max {st['max_err']:.2e} relL2 {st['rel_l2']:.2e}", flush=True)


# ------------------------------------------------------------------------ edge cases
def _small_cfg(cid, dtype, n_q=1, batch=1, fixed_len=40, H=4, d_c=32, d_r=8, d=16, rms=False):
    return MLAConfig(cid=cid, name="small", batch=batch, n_heads=H, d_model=64, q_lora=None, d_latent=d_c,
                     d_rope=d_r, d_nope=d, d_v=d, n_q=n_q, dtype=dtype, fixed_len=fixed_len, latent_rms_norm=rms)


def test_hand_worked_example_on_gpu():
    """The page's 3-token example run through the four calls (scale 1)."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "decoupled_rope_hand_example.json")) as f:
        g = json.load(f)
    cfg = _small_cfg(200, "f32", fixed_len=3, H=2, d_c=2, d_r=2, d=2)
    hi = host_inputs(cfg)
    hi.c = [np.array([[1, 0], [0, 1], [0.5, 0.5]], dtype=np.float32)]
    hi.k_pre = [np.asarray(g["expected_k_rope_pre"], dtype=np.float32)]
    hi.q_nope = np.array([[[[1, 0], [0, 1]]]], dtype=np.float32)
    hi.q_rope = np.asarray(g["expected_q_rope_pre"], dtype=np.float32)[None, None]
    hi.w_uk = np.asarray(g["constructed"]["w_uk"], dtype=np.float32)
    hi.w_uv = np.asarray(g["constructed"]["w_uv"], dtype=np.float32)
    run = run_pipeline(hi, scale=1.0)
    rows = np32(run.cache)
    assert np.max(np.abs(rows[:, 2:] - np.asarray(g["expected_k_rot"]))) <= g["printed_precision"]
    qp = np32(run.q_packed[0, 0])
    assert np.max(np.abs(qp[:, 2:] - np.asarray(g["expected_q_rot"]))) <= g["printed_precision"]
    # lse of the page's total scores (printed to 3 decimals, so 3 * 5e-4 slack)
    tot = np.asarray(g["expected_total_scores"])
    lse_page = np.log(np.exp(tot).sum(axis=1))
    assert np.max(np.abs(np32(run.lse[0, 0]) - lse_page)) <= 1.5e-3
    _check_outputs(run, hi, 0, scale=1.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_key_sequence(dtype):
    cfg = _small_cfg(201, dtype, fixed_len=1)
    hi = host_inputs(cfg)
    run = run_pipeline(hi)
    assert np.array_equal(np32(run.z[0, 0]), np.broadcast_to(hi.c[0][0].astype(np.float64), (4, 32)))
    _check_outputs(run, hi, 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_from_empty_cache(dtype):
    """n_q = seq_len: the square causal mask of a full forward."""
    cfg = _small_cfg(202, dtype, n_q=37, fixed_len=37)
    hi = host_inputs(cfg)
    run = run_pipeline(hi)
    _check_cache(run, hi, 0)
    _check_qpacked(run, hi, 0)
    _check_outputs(run, hi, 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_small_many_splits(dtype):
    cfg = _small_cfg(203, dtype, batch=5, fixed_len=None, n_q=3)
    cfg = MLAConfig(**{**cfg.__dict__, "ragged_range": (0, 300)})
    hi = host_inputs(cfg)
    run = run_pipeline(hi, n_splits=16)
    for b in range(5):
        _check_cache(run, hi, b)
        _check_outputs(run, hi, b)


def test_multi_step_decode_matches_oracle_each_step():
    """Append-then-attend over several consecutive tokens, one call sequence per token."""
    import mla_decode_decoupled_amd as mla
    cfg = _small_cfg(204, "f32", fixed_len=24)
    hi = host_inputs(cfg)
    lc = lib_config(cfg)
    H = cfg.n_heads
    n_total = 24
    cache = torch.full((n_total, cfg.row), float("nan"), dtype=torch.float32, device="cuda")
    seq_off = torch.zeros(1, dtype=torch.int64, device="cuda")
    qn_all = G._normal(cfg, G.TensorId.Q_NOPE, (n_total, H, cfg.d_nope), 1.0, 7)
    qr_all = G._normal(cfg, G.TensorId.Q_ROPE, (n_total, H, cfg.d_rope), 1.0, 7)
    w_uk, w_uv = tdev(hi.w_uk, torch.float32), tdev(hi.w_uv, torch.float32)
    for t in range(n_total):
        mla.mla_rope_append(lc, tdev(hi.c[0][None, t:t + 1], torch.float32),
                            tdev(hi.k_pre[0][None, t:t + 1], torch.float32), cache, seq_off,
                            torch.full((1,), t, dtype=torch.int32, device="cuda"))
        qp = torch.empty((1, H, cfg.row), dtype=torch.float32, device="cuda")
        mla.mla_absorb_q(lc, tdev(qn_all[t:t + 1], torch.float32), tdev(qr_all[t:t + 1], torch.float32),
                         torch.full((1,), t, dtype=torch.int32, device="cuda"), w_uk, qp)
        z = torch.empty((1, 1, H, cfg.d_latent), dtype=torch.float32, device="cuda")
        lse = torch.empty((1, 1, H), dtype=torch.float32, device="cuda")
        mla.mla_decode_attn(lc, qp.view(1, 1, H, cfg.row), cache, seq_off,
                            torch.full((1,), t + 1, dtype=torch.int32, device="cuda"), t + 1, z, lse)
        o = torch.empty((1, H, cfg.d_v), dtype=torch.float32, device="cuda")
        mla.mla_out_proj(lc, z.view(1, H, cfg.d_latent), w_uv, o)
        ref = O.explicit_attention(hi.c[0][:t + 1], hi.k_pre[0][:t + 1], qn_all[t:t + 1], qr_all[t:t + 1],
                                   hi.w_uk, hi.w_uv, scale=cfg.softmax_scale, base=cfg.rope_base)
        assert_close(np32(o)[0], ref["o"][0], "f32", f"o step {t}")
        assert_close(np32(z)[0, 0], ref["z"][0], "f32", f"z step {t}")


@pytest.mark.parametrize("n_splits", [0, 1, 3])
def test_later_scores_far_above_the_first_tile(n_splits):
    """A chunk whose later keys score far above its first tile (by more than 64 in log2 units)
    must still match the oracle: the fast kernel's fixed per-chunk reference cannot hold those
    probabilities, so it has to fall back to its exact online-softmax path.

    Construction (bf16 fast shape, 232 keys): keys 0..31 have zero latent and zero position key
    (score 0); keys 32.. all carry the same latent c* = sign(q~ of head 0), and every position
    part is zero. Head 0 then scores its later keys at scale * sum|q~| (about 100 in natural
    units), every other head at a moderate value; each head's softmax has two levels, which keeps
    the comparison well conditioned. n_splits = 0 takes the head-split kernel (chunks of two
    tiles): its first chunk falls back, for each block of 32 heads separately."""
    cfg = CONFIGS[1]
    n = 32 + 200
    hi = host_inputs(cfg, lens=[n])
    hi.q_rope = np.zeros_like(hi.q_rope)
    hi.k_pre = [np.zeros_like(hi.k_pre[0])]
    q_abs = O.absorb_query(hi.q_nope[0], hi.w_uk)[0]           # [H, d_c], row 0
    star = np.where(q_abs[0] >= 0, 1.0, -1.0).astype(np.float32)
    c = np.zeros((n, cfg.d_latent), np.float32)
    c[32:] = star
    hi.c = [c]
    scale = 0.5
    jump_log2 = scale * float(q_abs[0] @ star) * math.log2(math.e)
    assert jump_log2 > 2 * 64, f"construction must exceed the kernel's headroom: {jump_log2:.1f}"
    run = run_pipeline(hi, n_splits=n_splits, scale=scale)
    ref = _oracle(hi, 0, scale=scale)
    assert_close(np32(run.z[0]), ref["z"], cfg.dtype, "z")
    assert_close(np32(run.o[0]), ref["o"], cfg.dtype, "o")
    # lse reaches ~100 here, so it carries the score error of q_packed's bf16 storage:
    # |ds| <= scale * sum_c |q~_c c_c| * 2^-9 (half an ulp per element), on top of the usual bar.
    bound = scale * np.abs(q_abs) @ np.abs(star) * 2.0 ** -9 + 2e-2       # per head
    err = np.abs(np32(run.lse[0, 0]) - ref["lse"][0])
    assert np.all(err <= bound), f"lse: max err {err.max():.3e}, worst margin {(err - bound).max():.3e}"
    # head 0 puts all its weight on the later keys: z = c* up to exp(-jump)
    assert np.max(np.abs(np32(run.z[0, 0, 0]) - star)) <= 1e-3



def test_empty_work_is_a_noop():
    import mla_decode_decoupled_amd as mla
    from mla_decode_decoupled_amd import _lib
    cfg = lib_config(_small_cfg(205, "f32"))
    z = torch.full((1, 1, 4, 32), 7.0, device="cuda")
    st = _lib.lib.mla_decode_attn(cfg, 0, 1, None, None, None, None, 10, 0, None, 0, z.data_ptr(), None, None)
    assert st == _lib.MLA_OK
    st = _lib.lib.mla_rope_append(cfg, 3, 0, None, None, None, None, None, None)
    assert st == _lib.MLA_OK
    torch.cuda.synchronize()
    assert torch.all(z == 7.0)
