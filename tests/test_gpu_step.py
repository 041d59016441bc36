"""mla_decode_step, the four calls as one: through the C ABI it must write what mla_rope_append,
mla_absorb_q, mla_decode_attn and mla_out_proj write when called one after the other on the same
inputs — the cache rows and q_packed bit for bit; z, lse and o bit for bit too wherever the step
launches the single calls' kernels, and within float32 summation order (z, lse) and one bf16
rounding (o) where its split-K merge rides on the W_UV launch (few rows of the DeepSeek shape).
The outputs are also checked against the fp64 oracle, and the step is replayed from a captured
HIP graph."""

import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle as O  # noqa: E402
from mla_workloads import CONFIGS, MLAConfig  # noqa: E402

from .gpu_pipeline import (assert_close, host_inputs, lib_config, np32, run_pipeline, run_step,  # noqa: E402
                           tdev)

import mla_decode_decoupled_amd as mla  # noqa: E402


def _same(a: torch.Tensor, b: torch.Tensor, what: str):
    assert a.shape == b.shape, f"{what}: shape {tuple(a.shape)} vs {tuple(b.shape)}"
    if not torch.equal(a, b):
        d = (a.float() - b.float()).abs()
        raise AssertionError(f"{what}: step differs from the single calls (max |diff| {d.max().item():.3e}, "
                             f"{int((d > 0).sum().item())} elements)")


def _near(a: torch.Tensor, b: torch.Tensor, what: str, rel: float):
    """|a - b| <= rel * |b| + rel * max|b| elementwise (a reordered float32 sum, or a result
    rounded once more to bf16 from it)."""
    a64, b64 = a.double(), b.double()
    bound = rel * b64.abs() + rel * b64.abs().max()
    d = (a64 - b64).abs()
    assert bool((d <= bound).all()), f"{what}: max |diff| {d.max().item():.3e} beyond {rel:.1e} relative"


def _compare(hi, n_splits=0, scale=None, heads=(0, 31, 64, 127), fused_merge=False):
    ref = run_pipeline(hi, n_splits=n_splits, scale=scale)
    got = run_step(hi, n_splits=n_splits, scale=scale)
    for name in ("cache", "q_packed"):
        _same(getattr(got, name), getattr(ref, name), name)
    if fused_merge:
        _near(got.z, ref.z, "z", 1e-5)
        _near(got.lse, ref.lse, "lse", 1e-5)
        _near(got.o.float(), ref.o.float(), "o", 2.0 ** -7)
    else:
        for name in ("z", "lse", "o"):
            _same(getattr(got, name), getattr(ref, name), name)
    cfg = hi.cfg
    heads = [h for h in heads if h < cfg.n_heads]
    s = cfg.softmax_scale if scale is None else scale
    for b in sorted({0, len(hi.lens) - 1}):
        r = O.explicit_attention(hi.c[b], hi.k_pre[b], hi.q_nope[b], hi.q_rope[b], hi.w_uk, hi.w_uv,
                                 scale=s, base=cfg.rope_base, heads=heads)
        st = assert_close(np32(got.o[b])[:, heads], r["o"], cfg.dtype, f"step o[{b}]")
        assert_close(np32(got.z[b])[:, heads], r["z"], cfg.dtype, f"step z[{b}]")
        print(f"seq {b}: o max {st['max_err']:.2e} relL2 {st['rel_l2']:.2e}", flush=True)
    return got


def _v3(batch, n_q=1):
    return MLAConfig(**{**CONFIGS[1].__dict__, "batch": batch, "n_q": n_q})


def test_step_v3_decode_4k():
    """The batch-1 decode step of the DeepSeek-V3 shape over 4097 keys (the fused form)."""
    _compare(host_inputs(CONFIGS[1]), fused_merge=True)


def test_step_head_split_mixed_lengths():
    """Six query rows (3 sequences x 2): one row short enough for a single chunk, whose z the
    attention kernel writes itself and the fused projection reads back."""
    _compare(host_inputs(_v3(3, 2), lens=[41, 700, 3001]), fused_merge=True)


@pytest.mark.parametrize("batch", [15, 16], ids=["rows15_fused", "rows16_single_calls"])
def test_step_row_count_edges(batch):
    """15 rows is the largest fused step; at 16 the projections switch to the MFMA GEMMs and the
    step launches the single calls' kernels (positions written into its workspace)."""
    lens = np.random.default_rng(batch).integers(60, 1200, size=batch)
    _compare(host_inputs(_v3(batch), lens=lens), fused_merge=batch < 16)


@pytest.mark.parametrize("n_splits,lens", [(3, [900, 2500]), (0, [3000, 9000, 4100, 6000])],
                         ids=["fixed_splits", "balanced_plan"])
def test_step_without_head_split(n_splits, lens):
    """Few rows whose attention does not take the head-split kernel (a caller's split count, or
    histories too long for it): the step keeps the merge in the attention call."""
    _compare(host_inputs(_v3(len(lens)), lens=lens), n_splits=n_splits)


@pytest.mark.parametrize("batch,length", [(1, 32768), (1, 32769), (16, 2048), (16, 2049)],
                         ids=["b1_1024_tiles_hsplit", "b1_1025_tiles_balanced", "b16_64_tiles_hsplit",
                              "b16_65_tiles_balanced"])
def test_step_head_split_boundary(batch, length):
    """Both sides of the head-split kernel's limit (rows x tiles of the longest row <= 1024, at most
    16 rows). One key past it the balanced MFMA kernel and the single calls' merge take over. With
    fewer than 16 rows the step fuses the head-split merge into the W_UV launch; at 16 rows it runs
    the single calls' kernels either way. Equal lengths, so every row is at the bound."""
    hsplit = batch * ((length + 31) // 32) <= 1024
    _compare(host_inputs(_v3(batch), lens=[length] * batch), fused_merge=hsplit and batch < 16)


def test_step_chunked_rows():
    """Many query rows per sequence (chunked prefill): GEMM projections, MFMA attention."""
    _compare(host_inputs(_v3(2, 40), lens=[100, 300]))


def test_step_tiny_fp32():
    """The tiny fp32 workload: the generic kernels."""
    _compare(host_inputs(CONFIGS[0]))


def test_step_exact_fallback():
    """Later keys scoring far above a chunk's first tile: the head-split kernel's exact path
    writes its partials in the same head-major layout that the fused merge reads."""
    cfg = CONFIGS[1]
    n = 32 + 200
    hi = host_inputs(cfg, lens=[n])
    hi.q_rope = np.zeros_like(hi.q_rope)
    hi.k_pre = [np.zeros_like(hi.k_pre[0])]
    q_abs = O.absorb_query(hi.q_nope[0], hi.w_uk)[0]
    c = np.zeros((n, cfg.d_latent), np.float32)
    c[32:] = np.where(q_abs[0] >= 0, 1.0, -1.0)
    hi.c = [c]
    scale = 0.5
    assert scale * float(np.abs(q_abs[0]).sum()) * math.log2(math.e) > 2 * 64
    _compare(hi, scale=scale, heads=(1, 40, 100), fused_merge=True)


def test_step_graph_replay():
    """The step captured once and replayed: every replay (with eager steps and synchronisations
    in between) writes, bit for bit, what the eager step writes."""
    hi = host_inputs(_v3(2), lens=[500, 2048])
    cfg = hi.cfg
    lc = lib_config(cfg)
    dt = mla.storage_dtype(lc)
    B, H, R = 2, cfg.n_heads, 2
    eager = run_step(hi)
    lens = hi.lens
    c_new = tdev(np.stack([hi.c[b][int(lens[b]) - 1:] for b in range(B)]), dt)
    k_new = tdev(np.stack([hi.k_pre[b][int(lens[b]) - 1:] for b in range(B)]), dt)
    qn = tdev(hi.q_nope.reshape(R, H, cfg.d_nope), dt)
    qr = tdev(hi.q_rope.reshape(R, H, cfg.d_rope), dt)
    wuk, wuv = tdev(hi.w_uk, dt), tdev(hi.w_uv, dt)
    cache = eager.cache.clone()
    qp = torch.empty_like(eager.q_packed).view(R, H, cfg.row)
    z, lse = torch.empty_like(eager.z), torch.empty_like(eager.lse)
    o = torch.empty((R, H, cfg.d_v), dtype=dt, device="cuda")
    max_len = int(lens.max())
    ws = torch.empty(mla.mla_decode_step_workspace_size(lc, B, 1, max_len), dtype=torch.uint8, device="cuda")

    def step():
        mla.mla_decode_step(lc, c_new, k_new, qn, qr, wuk, wuv, cache, eager.seq_off, eager.seq_len, max_len,
                            qp, z, o, lse=lse, workspace=ws)

    step()   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for k in range(3):
        for t in (z, lse, o, qp):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _same(z, eager.z, f"replay {k} z")
        _same(lse, eager.lse, f"replay {k} lse")
        _same(o, eager.o.view(R, H, cfg.d_v), f"replay {k} o")
        _same(qp, eager.q_packed.view(R, H, cfg.row), f"replay {k} q_packed")
        _same(cache, eager.cache, f"replay {k} cache")
        step()   # eager work between replays
        torch.cuda.synchronize()
