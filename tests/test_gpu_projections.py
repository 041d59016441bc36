"""GPU parity of the upstream projections (mla_project_kv_append, mla_project_q) and of the
decode advance, through the C ABI, against the fp64 oracle on the same seeded inputs."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
from mla_workloads import MLAConfig, get_config  # noqa: E402
from mla_workloads import generate as G  # noqa: E402

from .gpu_pipeline import assert_close, lib_config, np32, tdev  # noqa: E402

import mla_decode_decoupled_amd as mla  # noqa: E402

PROJ_KEYS = ("w_dkv", "w_kr", "kv_norm_w", "w_q", "w_dq", "w_uq", "w_qr")


def _tiny(q_lora, norm, cid):
    base = get_config(0)
    return MLAConfig(cid=cid, name="tiny_proj", batch=2, n_heads=base.n_heads, d_model=base.d_model, q_lora=q_lora,
                     d_latent=base.d_latent, d_rope=base.d_rope, d_nope=base.d_nope, d_v=base.d_v, n_q=1,
                     dtype="f32", fixed_len=8, latent_rms_norm=norm)


def _run_kv(cfg, w, h, len_before, eps=1e-6):
    """h [B, n_new, d_model] host; returns the device cache and the oracle's rows per token."""
    lc = lib_config(cfg)
    dt = mla.storage_dtype(lc)
    B, n_new, dm = h.shape
    cap = int(len_before.max()) + n_new + 3
    cache = torch.full((B * cap, cfg.row), float("nan"), dtype=dt, device="cuda")
    seq_off = torch.arange(B, dtype=torch.int64, device="cuda") * cap
    lb = torch.from_numpy(len_before.astype(np.int32)).cuda()
    ws = torch.empty(mla.mla_project_workspace_size(lc, B * n_new, dm, 0), dtype=torch.uint8, device="cuda")
    norm = tdev(w["kv_norm_w"], dt) if "kv_norm_w" in w else None
    w_kr = tdev(w["w_kr"], dt)
    w_kr_copy = w_kr.clone()
    mla.mla_project_kv_append(lc, tdev(h, dt), tdev(w["w_dkv"], dt), w_kr, cache, seq_off, lb,
                              kv_norm_w=norm, kv_norm_eps=eps, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(w_kr, w_kr_copy)
    got, ref = [], []
    weights = {k: w[k] for k in PROJ_KEYS if k in w}
    for b in range(B):
        p = O.project_inputs(h[b], weights, cfg.n_heads, kv_norm_eps=eps)
        pos = int(len_before[b]) + np.arange(n_new)
        ref.append(O.cache_rows(p["c"], p["k_rope_pre"], pos, cfg.rope_base))
        got.append(np32(cache[b * cap + pos[0]: b * cap + pos[-1] + 1]))
        # rows outside the written range stay untouched
        untouched = np32(cache[b * cap: b * cap + pos[0]])
        assert np.all(np.isnan(untouched))
    return np.concatenate(got), np.concatenate(ref)


def _run_q(cfg, w, h):
    lc = lib_config(cfg)
    dt = mla.storage_dtype(lc)
    R, dm = h.shape
    H = cfg.n_heads
    d_q = cfg.q_lora or 0
    qn = torch.full((R, H, cfg.d_nope), float("nan"), dtype=dt, device="cuda")
    qr = torch.full((R, H, cfg.d_rope), float("nan"), dtype=dt, device="cuda")
    ws = torch.empty(mla.mla_project_workspace_size(lc, R, dm, d_q), dtype=torch.uint8, device="cuda")
    w_uq = w["w_uq"] if d_q else w["w_q"]
    mla.mla_project_q(lc, tdev(h, dt), tdev(w_uq, dt), tdev(w["w_qr"], dt), qn, qr,
                      w_dq=tdev(w["w_dq"], dt) if d_q else None, workspace=ws)
    torch.cuda.synchronize()
    p = O.project_inputs(h, {k: w[k] for k in PROJ_KEYS if k in w}, H)
    return np32(qn), np32(qr), p["q_nope"], p["q_rope_pre"]


@pytest.mark.parametrize("norm", [False, True], ids=["plain", "rmsnorm"])
def test_project_kv_append_tiny_fp32(norm):
    cfg = _tiny(None, norm, 90 + int(norm))
    w = G.full_layer_inputs(cfg, 6)
    h = w["h"].reshape(2, 3, cfg.d_model)
    got, ref = _run_kv(cfg, w, h, np.array([5, 17]))
    assert_close(got, ref, "f32", f"cache rows (norm={norm})")


@pytest.mark.parametrize("q_lora", [None, 48], ids=["direct", "compressed"])
def test_project_q_tiny_fp32(q_lora):
    cfg = _tiny(q_lora, False, 92 + (q_lora or 0))
    w = G.full_layer_inputs(cfg, 5)
    qn, qr, qn_ref, qr_ref = _run_q(cfg, w, w["h"])
    assert_close(qn, qn_ref, "f32", "q_nope")
    assert_close(qr, qr_ref, "f32", "q_rope (unrotated)")


@pytest.fixture(scope="module")
def v3_weights():
    cfg = get_config(1)
    w = G.full_layer_inputs(cfg, 520)
    w.pop("w_o")
    return cfg, w


# 1-5 rows: the matrix-vector kernel (row blocks of 1, 2 and 4, with a ragged tail);
# 16, 160 and 520 rows: the MFMA GEMM (one partial row tile, a ragged second tile, five tiles)
@pytest.mark.parametrize("rows", [1, 2, 3, 5, 16, 160, 520])
def test_project_v3_shape_bf16(v3_weights, rows):
    cfg, w = v3_weights
    h = w["h"][:rows]
    qn, qr, qn_ref, qr_ref = _run_q(cfg, w, h)
    s1 = assert_close(qn, qn_ref, "bf16", f"q_nope rows={rows}")
    s2 = assert_close(qr, qr_ref, "bf16", f"q_rope rows={rows}")
    # the kv side: as one sequence of `rows` new tokens after 100 cached ones, and as `rows`
    # sequences of one token each at scattered positions
    got, ref = _run_kv(cfg, w, h[None], np.array([100]))
    s3 = assert_close(got, ref, "bf16", f"cache rows rows={rows} (one sequence)")
    if rows <= 160:
        lb = np.random.default_rng(rows).integers(0, 5000, size=rows)
        got, ref = _run_kv(cfg, w, h[:, None], lb)
        assert_close(got, ref, "bf16", f"cache rows rows={rows} (one token per sequence)")
    print(f"rows={rows} q_nope {s1} q_rope {s2} cache {s3}")


def test_decode_advance_moves_positions():
    lb = torch.tensor([0, 7, 100], dtype=torch.int32, device="cuda")
    sl = torch.tensor([1, 8, 101], dtype=torch.int32, device="cuda")
    qp = torch.tensor([0, 7, 100, 3, 9], dtype=torch.int32, device="cuda")
    mla.mla_decode_advance(2, len_before=lb, seq_len=sl, q_pos=qp)
    mla.mla_decode_advance(1, seq_len=sl)
    torch.cuda.synchronize()
    assert lb.tolist() == [2, 9, 102]
    assert sl.tolist() == [4, 11, 104]
    assert qp.tolist() == [2, 9, 102, 5, 11]


def _run_inputs(cfg, w, h, len_before, eps=1e-6):
    """mla_project_inputs on h [B, n_new, d_model]: the cache rows per token and the query outputs."""
    lc = lib_config(cfg)
    dt = mla.storage_dtype(lc)
    B, n_new, dm = h.shape
    R, H = B * n_new, cfg.n_heads
    d_q = cfg.q_lora or 0
    cap = int(len_before.max()) + n_new + 3
    cache = torch.full((B * cap, cfg.row), float("nan"), dtype=dt, device="cuda")
    seq_off = torch.arange(B, dtype=torch.int64, device="cuda") * cap
    lb = torch.from_numpy(len_before.astype(np.int32)).cuda()
    qn = torch.full((R, H, cfg.d_nope), float("nan"), dtype=dt, device="cuda")
    qr = torch.full((R, H, cfg.d_rope), float("nan"), dtype=dt, device="cuda")
    ws = torch.empty(mla.mla_project_inputs_workspace_size(lc, R, dm, d_q), dtype=torch.uint8, device="cuda")
    norm = tdev(w["kv_norm_w"], dt) if "kv_norm_w" in w else None
    w_uq = w["w_uq"] if d_q else w["w_q"]
    mla.mla_project_inputs(lc, tdev(h, dt), tdev(w["w_dkv"], dt), tdev(w["w_kr"], dt), cache, seq_off, lb,
                           tdev(w_uq, dt), tdev(w["w_qr"], dt), qn, qr,
                           w_dq=tdev(w["w_dq"], dt) if d_q else None, kv_norm_w=norm, kv_norm_eps=eps, workspace=ws)
    torch.cuda.synchronize()
    weights = {k: w[k] for k in PROJ_KEYS if k in w}
    got, ref = [], []
    for b in range(B):
        p = O.project_inputs(h[b], weights, H, kv_norm_eps=eps)
        pos = int(len_before[b]) + np.arange(n_new)
        ref.append(O.cache_rows(p["c"], p["k_rope_pre"], pos, cfg.rope_base))
        got.append(np32(cache[b * cap + pos[0]: b * cap + pos[-1] + 1]))
        assert np.all(np.isnan(np32(cache[b * cap: b * cap + pos[0]])))
    pq = O.project_inputs(h.reshape(R, dm), weights, H)
    return np.concatenate(got), np.concatenate(ref), np32(qn), np32(qr), pq["q_nope"], pq["q_rope_pre"]


# 1-15 rows: the two-launch form (h read once for W_DKV, W_KR and W_DQ; the kv finish on the
# W_UQ / W_QR launch), 16 rows: the four launches of the separate calls
@pytest.mark.parametrize("batch,n_new", [(1, 1), (3, 1), (5, 3), (16, 1)])
def test_project_inputs_v3_shape_bf16(v3_weights, batch, n_new):
    cfg, w = v3_weights
    h = w["h"][:batch * n_new].reshape(batch, n_new, cfg.d_model)
    lb = np.random.default_rng(batch * 7 + n_new).integers(0, 3000, size=batch)
    got, ref, qn, qr, qn_ref, qr_ref = _run_inputs(cfg, w, h, lb)
    s1 = assert_close(got, ref, "bf16", f"cache rows B={batch} n_new={n_new}")
    s2 = assert_close(qn, qn_ref, "bf16", "q_nope")
    s3 = assert_close(qr, qr_ref, "bf16", "q_rope (unrotated)")
    print(f"B={batch} n_new={n_new}: cache {s1} q_nope {s2} q_rope {s3}")


@pytest.mark.parametrize("q_lora,norm", [(None, True), (48, False)], ids=["direct_rmsnorm", "compressed_plain"])
def test_project_inputs_tiny_fp32(q_lora, norm):
    cfg = _tiny(q_lora, norm, 94 + (q_lora or 0) + int(norm))
    w = G.full_layer_inputs(cfg, 6)
    got, ref, qn, qr, qn_ref, qr_ref = _run_inputs(cfg, w, w["h"].reshape(2, 3, cfg.d_model), np.array([4, 11]))
    assert_close(got, ref, "f32", "cache rows")
    assert_close(qn, qn_ref, "f32", "q_nope")
    assert_close(qr, qr_ref, "f32", "q_rope (unrotated)")
