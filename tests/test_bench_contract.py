"""CPU checks of bench.py's command-line contract that need no GPU: the build runs on one GPU, so any
other --gpus value ends the run with a message and a failing status before a device is touched; the
traffic records it reads are keyed by the current kernel sources; and the CPU-baseline leg's parity
field compares the oracle's outputs with the result it is handed."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                         text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert line["n_gpus_requested"] == n and "one GPU" in line["error"]


def test_traffic_records_parse():
    """Every record of the committed counter summary names a workload, a call, a split count, a source
    hash and a positive byte count; records whose hash matches the sources are found by the lookup."""
    sys.path.insert(0, ROOT)
    import bench

    text = open(bench.COUNTERS_FILE).read()
    recs = json.loads(text.split("```json", 1)[1].split("```", 1)[0])["records"]
    assert recs
    sha = bench.sources_sha()
    for r in recs:
        assert r["traffic_bytes_per_call"] > 0 and len(r["source_sha"]) == 16
        got = bench.recorded_traffic(r["workload"], r["call"], r["n_splits"], cold=True)
        assert got == (r["traffic_bytes_per_call"] if r["source_sha"] == sha else None)
        assert bench.recorded_traffic(r["workload"], r["call"], r["n_splits"], cold=False) is None


def test_source_hash_follows_code_not_comments(tmp_path):
    """The records' key hashes the code only: a comment or blank-line edit keeps it, a code edit changes it."""
    sys.path.insert(0, ROOT)
    import bench

    code = "int f(int a) {\n  return a + 1;\n}\n"
    a = tmp_path / "a.hip"
    a.write_text(code)
    b = tmp_path / "b.hip"
    b.write_text("// header\n/* a block\n   comment */\nint f(int a) {   \n\n  return a + 1;  // one more\n}\n")
    c = tmp_path / "c.hip"
    c.write_text(code.replace("a + 1", "a + 2"))
    assert bench.sources_sha([str(a)]) == bench.sources_sha([str(b)])
    assert bench.sources_sha([str(a)]) != bench.sources_sha([str(c)])


def _host_workload(cid):
    """The host half of bench.Workload for workload `cid` (inputs drawn, nothing on a device)."""
    import numpy as np
    import torch

    from mla_workloads import get_config
    from mla_workloads import generate as G

    cfg = get_config(cid)
    lens = G.seq_lens(cfg)
    B, n_q, H = cfg.batch, cfg.n_q, cfg.n_heads

    class W:
        pass

    W.cfg, W.lens, W.B, W.n_q, W.H, W.R = cfg, lens, B, n_q, H, B * n_q
    W.c_host = [G.cache_latent(cfg, b, int(lens[b])) for b in range(B)]
    W.k_host = [G.cache_rope_pre(cfg, b, int(lens[b])) for b in range(B)]
    W.qn_host = np.stack([G.query_nope(cfg, b) for b in range(B)]).reshape(B * n_q, H, cfg.d_nope)
    W.qr_host = np.stack([G.query_rope_pre(cfg, b) for b in range(B)]).reshape(B * n_q, H, cfg.d_rope)
    W.wuk_host, W.wuv_host = G.weight_uk(cfg), G.weight_uv(cfg)
    W.z = torch.zeros((B, n_q, H, cfg.d_latent), dtype=torch.float32)
    W.o = torch.zeros((B * n_q, H, cfg.d_v), dtype=torch.float32)
    return W


def test_cpu_baseline_parity_field():
    """The CPU-baseline leg compares the oracle's outputs for the heads it evaluates with the device
    result it is handed (here a host tensor): a result equal to the oracle's passes, every head is
    checked, and a result off by more than the tolerance in one element fails."""
    sys.path.insert(0, ROOT)
    import bench
    import oracle as O

    W = _host_workload(0)
    cfg = W.cfg
    ref = O.explicit_attention(W.c_host[0], W.k_host[0], W.qn_host, W.qr_host, W.wuk_host, W.wuv_host,
                               scale=cfg.softmax_scale, base=cfg.rope_base)
    import torch

    W.z[0] = torch.from_numpy(ref["z"].astype("float32"))
    out = bench.cpu_baseline(W, 0.3)["parity"]
    assert out["pass"] and out["heads_checked"] == cfg.n_heads and out["max_abs_err"] < 1e-6
    W.z[0, 0, cfg.n_heads - 1, 3] += 1e-3
    out = bench.cpu_baseline(W, 0.3)["parity"]
    assert not out["pass"] and out["max_abs_err"] > 5e-4


def test_stamp_summary_phases():
    """bench.py's reading of the phase stamps (slot layout of include/mla_stamps.h) on two synthetic
    workgroups at 2 GHz: phase lengths, cycles per tile, and the start and end spreads on the 100 MHz
    counter; inactive workgroups (exit slot 0) are left out."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import bench

    st = np.zeros((8192, 16), dtype=np.uint64)
    for wg, (start, tiles) in enumerate([(1000, 10), (1100, 20)]):
        t0 = 5_000_000
        cyc = [t0, t0 + 2000, t0 + 6000, t0 + 10000, t0 + 10000 + 3000 * tiles, t0 + 12000 + 3000 * tiles]
        st[wg, :6] = cyc
        st[wg, 8] = start
        st[wg, 9] = start + (cyc[5] - cyc[0]) // 20          # 2 GHz against 100 MHz: 20 cycles a tick
        st[wg, 10], st[wg, 11], st[wg, 12], st[wg, 13] = tiles, 0, wg, 1
    st[2, 0], st[2, 13] = 7, 1                               # started, never finished: left out
    out = bench.stamp_summary(st)
    assert out["workgroups"] == 2 and out["kernel"] == "decode_attn_fast"
    assert abs(out["clock_ghz_median"] - 2.0) < 1e-9
    assert out["chunk_plan_us"]["median"] == 1.0 and out["queries_to_registers_us"]["median"] == 2.0
    assert out["cycles_per_tile_median"] == 3000.0
    assert out["start_spread_us"] == 1.0
    # ends: 1000 + (42000 / 20) and 1100 + (72000 / 20) ticks
    assert out["end_spread_us"] == round(((1100 + 3600) - (1000 + 2100)) / 100.0, 2)
