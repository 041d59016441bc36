#!/usr/bin/env python3
"""Benchmark of one absorbed-MLA decode step on one MI355X.

A step is one pass of the whole hot path over one batch: the append of the new
tokens, the query absorption, the latent attention (+ split-K merge) and the
W_UV projection, through the C ABI as one mla_decode_step call (three launches
at batch 1), or with --single-calls as mla_rope_append, mla_absorb_q,
mla_decode_attn and mla_out_proj. The default workload is the DeepSeek-V3-shaped decode
step (batch 1, 128 heads, 512-dim latent, 64-dim position part, 4096 cached
tokens + 1 new, bf16). Inputs are seeded synthetic data of that shape and live
in HBM before timing starts. Unless --hot is given, every step reads its own
copy of the cache, weights and queries (copies rotated so the working set is
at least 1 GiB, four times the 256 MB last-level cache), so the bytes really
come from HBM. The timed steps replay one captured HIP graph per input copy
(--eager launches them from Python instead, which is bound by the launch
overhead at batch 1); the eager time is reported too. A second pass runs the
four single calls with HIP events between them for the per-call times.

Prints one JSON line (rank 0) with throughput, a roofline object for the
dominant call (mla_decode_attn: HIP events around it in the per-call pass) and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1, help="workload id (1 = V3 decode, batch 1, S=4096)")
    ap.add_argument("--n-splits", type=int, default=0, help="split-K chunks per sequence (0 = library choice)")
    ap.add_argument("--hot", action="store_true", help="reuse one copy of every input (cache-hot numbers)")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0 = enough for 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget for the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch the four calls from Python every step instead of replaying a captured HIP graph")
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--single-calls", action="store_true",
                    help="time the step as the four single calls instead of one mla_decode_step")
    ap.add_argument("--explicit", action="store_true",
                    help="many-row workloads: the step is mla_rope_append + mla_prefill_explicit (the non-absorbed "
                         "form) instead of absorb + latent attention + W_UV")
    ap.add_argument("--merged-wo-check", action="store_true",
                    help="time the output side at batch 1 both ways: W_UV per head then W_O (the library's "
                         "path) against one pre-merged [d_model x H*d_latent] matrix W_O W_UV applied to z")
    ap.add_argument("--decode-loop", action="store_true",
                    help="instead of the single step: time token-by-token decode through a stack of full MLA "
                         "layers (h -> projections -> attention -> W_O) replayed as one HIP graph per token")
    ap.add_argument("--layers", type=int, default=61, help="--decode-loop: layers in the stack")
    ap.add_argument("--loop-context", type=int, default=4096, help="--decode-loop: tokens prefilled per sequence")
    ap.add_argument("--loop-batch", type=int, default=1, help="--decode-loop: sequences decoded together")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the step: time a plain 1 GiB device copy (the reference kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return ap.parse_args()


COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_attn_v3_decode_s4k_counters.md")
TRAFFIC_SOURCES = [os.path.join(ROOT, "mla_decode_decoupled_amd", "csrc", f)
                   for f in ("api.hip", "generic.hip", "decode_fast.hip")]


def sources_sha() -> str:
    """Hash of the sources that decide what the attention kernels read and write."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, n_splits: int, cold: bool):
    """HBM bytes per mla_decode_attn call from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by the plain-copy calibration), or None when the summary is missing,
    was taken on another workload, or the kernels changed since it was taken."""
    try:
        text = open(COUNTERS_FILE).read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)
    except (OSError, IndexError, ValueError):
        return None
    if (rec.get("workload") != workload or rec.get("n_splits") != n_splits or not cold
            or rec.get("source_sha") != sources_sha()):
        return None
    return rec.get("traffic_bytes_per_call")


def copy_calibration(args):
    """One plain device-to-device copy kernel of known size, repeated: the counters read for it
    give the factor between FETCH_SIZE / WRITE_SIZE and the bytes really moved."""
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    reps = 5
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps, "ms_per_copy": round(ms, 4),
                      "gbs_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args)
        return
    if args.decode_loop:
        decode_loop(args)
        return
    if args.merged_wo_check:
        merged_wo_check(args)
        return

    import numpy as np
    import torch

    import mla_decode_decoupled_amd as mla
    from mla_workloads import get_config
    from mla_workloads import generate as G

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = get_config(args.config)
    lc = mla.make_config(cfg.n_heads, cfg.d_nope, cfg.d_latent, cfg.d_rope, cfg.d_v, cfg.dtype, cfg.rope_base)
    dt = mla.storage_dtype(lc)
    esz = 2 if cfg.dtype == "bf16" else 4
    B, n_q, H, row = cfg.batch, cfg.n_q, cfg.n_heads, cfg.row
    lens = G.seq_lens(cfg)
    R = B * n_q
    max_len = int(lens.max())
    n_splits = args.n_splits or cfg.n_splits

    # ------------------------------------------------------------------ inputs (host, seeded)
    t0 = time.time()
    c_host = [G.cache_latent(cfg, b, int(lens[b])) for b in range(B)]
    k_host = [G.cache_rope_pre(cfg, b, int(lens[b])) for b in range(B)]
    qn_host = np.stack([G.query_nope(cfg, b) for b in range(B)]).reshape(R, H, cfg.d_nope)
    qr_host = np.stack([G.query_rope_pre(cfg, b) for b in range(B)]).reshape(R, H, cfg.d_rope)
    wuk_host, wuv_host = G.weight_uk(cfg), G.weight_uv(cfg)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)  # noqa: E731

    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    seq_off = torch.from_numpy(offs).to(dev)
    seq_len = torch.from_numpy(lens.astype(np.int32)).to(dev)
    len_before = torch.from_numpy((lens - n_q).astype(np.int32)).to(dev)
    q_pos = torch.from_numpy(np.concatenate([np.arange(int(l) - n_q, int(l)) for l in lens]).astype(np.int32)).to(dev)
    c_new = up(np.stack([c_host[b][int(lens[b]) - n_q:] for b in range(B)]))
    k_new = up(np.stack([k_host[b][int(lens[b]) - n_q:] for b in range(B)]))

    # one copy: cache (history appended by the library itself), weights, queries
    cache0 = torch.empty((int(lens.sum()), row), dtype=dt, device=dev)
    for b in range(B):
        h = int(lens[b]) - n_q
        if h > 0:
            mla.mla_rope_append(lc, up(c_host[b][None, :h]), up(k_host[b][None, :h]), cache0, seq_off[b:b + 1],
                                torch.zeros(1, dtype=torch.int32, device=dev))
    wuk0, wuv0 = up(wuk_host), up(wuv_host)
    qn0, qr0 = up(qn_host), up(qr_host)
    per_copy = (cache0.numel() + wuk0.numel() + wuv0.numel() + qn0.numel() + qr0.numel()) * esz
    if args.hot:
        n_copies = 1
    else:
        n_copies = args.copies or max(1, min(64, math.ceil((1 << 30) / per_copy)))
    copies = [(cache0, wuk0, wuv0, qn0, qr0)]
    for _ in range(n_copies - 1):
        copies.append(tuple(t.clone() for t in copies[0]))
    # outputs and workspace (shared by all copies)
    q_packed = torch.empty((R, H, row), dtype=dt, device=dev)
    z = torch.empty((B, n_q, H, cfg.d_latent), dtype=torch.float32, device=dev)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev)
    o = torch.empty((R, H, cfg.d_v), dtype=dt, device=dev)
    if args.explicit:
        ws_bytes = mla.mla_prefill_explicit_workspace_size(lc, B, n_q, max_len)
        if ws_bytes == 0:
            raise SystemExit("--explicit needs the bf16 DeepSeek head shape and n_q <= keys")
    else:
        ws_bytes = mla.mla_decode_attn_workspace_size(lc, B, n_q, max_len, n_splits)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    ws_step = None
    if not args.explicit:
        ws_step = torch.empty(mla.mla_decode_step_workspace_size(lc, B, n_q, max_len, n_splits), dtype=torch.uint8,
                              device=dev)
    fused = not args.explicit and not args.single_calls
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    stream = torch.cuda.current_stream(dev)
    ev = {k: [] for k in ("append", "absorb", "attn", "proj")}

    def step(i, timed):
        cache, wuk, wuv, qn, qr = copies[i % n_copies]
        if fused and not timed:
            # the four calls as one (two launches fewer for few rows); the per-call timing pass
            # below runs them one by one to time each
            mla.mla_decode_step(lc, c_new, k_new, qn, qr, wuk, wuv, cache, seq_off, seq_len, max_len, q_packed,
                                z, o, lse=lse, n_splits=n_splits, workspace=ws_step)
            return
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if timed else None
        if timed:
            marks[0].record(stream)
        mla.mla_rope_append(lc, c_new, k_new, cache, seq_off, len_before)
        if timed:
            marks[1].record(stream)
        if args.explicit:
            # the non-absorbed form: keys and values rebuilt from the cache, o written directly
            if timed:
                marks[2].record(stream)
            mla.mla_prefill_explicit(lc, qn.view(B, n_q, H, cfg.d_nope), qr.view(B, n_q, H, cfg.d_rope), cache,
                                     seq_off, seq_len, max_len, wuk, wuv, o.view(B, n_q, H, cfg.d_v), lse=lse,
                                     workspace=ws)
            if timed:
                marks[3].record(stream)
                marks[4].record(stream)
                for j, k in enumerate(("append", "absorb", "attn", "proj")):
                    ev[k].append((marks[j], marks[j + 1]))
            return
        mla.mla_absorb_q(lc, qn, qr, q_pos, wuk, q_packed)
        if timed:
            marks[2].record(stream)
        mla.mla_decode_attn(lc, q_packed.view(B, n_q, H, row), cache, seq_off, seq_len, max_len, z, lse,
                            n_splits=n_splits, workspace=ws)
        if timed:
            marks[3].record(stream)
        mla.mla_out_proj(lc, z.view(R, H, cfg.d_latent), wuv, o)
        if timed:
            marks[4].record(stream)
            for j, k in enumerate(("append", "absorb", "attn", "proj")):
                ev[k].append((marks[j], marks[j + 1]))

    for i in range(max(args.warmup, n_copies)):
        step(i, False)
    torch.cuda.synchronize()

    def time_steps(run):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(args.steps):
            run(i)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    # Eager launches cost ~10 us of Python and HIP API time per call, more than the batch-1 GPU work,
    # so a serving loop captures its work once per buffer set and replays it. Here: one HIP graph per
    # input copy (one step each), and one graph holding one step per copy in rotation order — the
    # same calls with the same kernels, recorded back to back the way a model's layers share one
    # graph, so a replay launch is paid once per rotation instead of once per step. The timed
    # steps replay the rotation graph and finish with single-step graphs; ms_per_step_graph1 is
    # the time when every step is a graph launch of its own.
    ms_step_eager = time_steps(lambda i: step(i, False))
    ms_step = ms_step_eager
    ms_step_graph1 = None
    if not args.eager:
        graphs = []
        for i in range(n_copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i, False)
            graphs.append(g)
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for i in range(n_copies):
                step(i, False)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % n_copies].replay()
        g_all.replay()
        torch.cuda.synchronize()
        ms_step_graph1 = time_steps(lambda i: graphs[i % n_copies].replay())

        def rotations(i):
            # called once per timed step: a rotation graph at every n_copies-th step while whole
            # rotations remain, single-step graphs for the rest
            full = args.steps // n_copies
            if i < full * n_copies:
                if i % n_copies == 0:
                    g_all.replay()
            else:
                graphs[i % n_copies].replay()
        ms_step = time_steps(rotations)
    # Per-call timing pass (events between the calls), same rotation. A spin kernel ahead of each
    # step keeps the GPU busy while Python enqueues the step, so the intervals are GPU time only.
    for i in range(args.steps):
        torch.cuda._sleep(400_000)
        step(i, True)
    torch.cuda.synchronize()
    per_kernel_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}

    # ------------------------------------------------------------------ algorithmic work
    keys = int(lens.sum())
    if n_q == 1:
        vis_pairs = keys
    else:
        vis_pairs = int(sum(n_q * (int(l) - n_q) + n_q * (n_q + 1) // 2 for l in lens))
    attn_bytes = keys * row * esz + R * H * row * esz + R * H * cfg.d_latent * 4 + R * H * 4
    attn_flops = 2 * H * (row + cfg.d_latent) * vis_pairs
    if args.explicit:
        # per (row, key, head): 192-wide scores and 128-wide values; plus rebuilding K_C and V per key;
        # bytes: cache rows, the rebuilt keys and values written and read once, queries in, o out
        attn_flops = (2 * H * (cfg.d_nope + cfg.d_rope + cfg.d_v) * vis_pairs
                      + 2 * keys * cfg.d_latent * H * (cfg.d_nope + cfg.d_v))
        attn_bytes = (keys * row * esz + 2 * keys * H * (cfg.d_nope + cfg.d_v) * esz
                      + 2 * H * cfg.d_nope * cfg.d_latent * esz
                      + R * H * (cfg.d_nope + cfg.d_rope) * esz + R * H * cfg.d_v * esz + R * H * 4)
    kernel_bytes = {
        "append": R * (cfg.d_latent + cfg.d_rope) * esz + R * row * esz,
        "absorb": H * cfg.d_nope * cfg.d_latent * esz + R * H * (cfg.d_nope + cfg.d_rope) * esz + R * H * row * esz,
        "attn": attn_bytes,
        "proj": H * cfg.d_v * cfg.d_latent * esz + R * H * cfg.d_latent * 4 + R * H * cfg.d_v * esz,
    }
    dominant = max(per_kernel_ms, key=per_kernel_ms.get)
    if dominant == "attn":
        t_bw, t_mf = attn_bytes / (HBM_PEAK_GBS * 1e9), attn_flops / (BF16_PEAK_TFLOPS * 1e12)
        bound = "hbm" if t_bw >= t_mf else "mfma"
    else:
        bound = "hbm"
    dom_s = per_kernel_ms[dominant] * 1e-3
    if bound == "hbm":
        achieved, peak, unit = kernel_bytes[dominant] / dom_s / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = attn_flops / dom_s / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"

    tokens_per_s = R / (ms_step * 1e-3)

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, c_host, k_host, qn_host, qr_host, wuk_host, wuv_host, lens, args.cpu_seconds)

    out = {
        "metric": "MLA decode tokens/s + achieved HBM GB/s (H=128, d_c=512, S=4K-128K)",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "ms_per_step_eager": round(ms_step_eager, 6),
        "ms_per_step_graph1": None if ms_step_graph1 is None else round(ms_step_graph1, 6),
        "launch": "eager" if args.eager else "hip_graph",
        "step_call": ("mla_prefill_explicit" if args.explicit
                      else "mla_decode_step" if fused else "four single calls"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) inputs, N(0,1/fan_in) weights, RMS-normalised latent)",
        "config": {"workload": cfg.name + ("_explicit" if args.explicit else ""), "batch": B, "n_q": n_q, "heads": H, "d_latent": cfg.d_latent,
                   "d_rope": cfg.d_rope, "d_nope": cfg.d_nope, "d_v": cfg.d_v,
                   "seq_len_keys": int(max_len) if len(set(lens.tolist())) == 1 else [int(lens.min()), int(lens.max())],
                   "n_splits": n_splits, "cold_copies": n_copies, "parallelism": "single GPU"},
        "roofline": {"kernel": {"attn": "mla_prefill_explicit" if args.explicit else "mla_decode_attn",
                                "absorb": "mla_absorb_q", "proj": "mla_out_proj",
                                "append": "mla_rope_append"}[dominant],
                     "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": (recorded_traffic(cfg.name, n_splits, not args.hot)
                                 if dominant == "attn" and not args.explicit else None),
                     "algorithmic_bytes_per_launch": kernel_bytes[dominant],
                     "avg_launch_ms": round(per_kernel_ms[dominant], 6)},
        "kernels_ms": {k: round(v, 6) for k, v in per_kernel_ms.items()},
        "attn_gbs": round(attn_bytes / (per_kernel_ms["attn"] * 1e-3) / 1e9, 2),
        "attn_tflops": round(attn_flops / (per_kernel_ms["attn"] * 1e-3) / 1e12, 3),
        "cpu_baseline": cpu,
    }
    if args.verbose:
        print(f"setup {setup_s:.1f}s, copies {n_copies} x {per_copy / 1e6:.1f} MB", file=sys.stderr)
    print(json.dumps(out), flush=True)


def decode_loop(args):
    """Per-token latency of a stack of DeepSeek-V3-shaped MLA layers at batch B: every layer runs
    mla_project_kv_append, mla_project_q, mla_absorb_q, mla_decode_attn and mla_out_proj with W_O,
    the layer's output feeding the next layer; the caches are first filled by a prefill of
    --loop-context tokens through the same stack, then one captured decode step (all layers and
    the position advance) is replayed per token. The weights of 61 layers (~23 GB) are far beyond
    the last-level cache, so every token streams them from HBM."""
    import torch

    import mla_decode_decoupled_amd as mla
    from mla_decode_decoupled_amd.decode_loop import DecodeStack, random_layers
    from mla_workloads import get_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = get_config(1)
    lc = mla.make_config(cfg.n_heads, cfg.d_nope, cfg.d_latent, cfg.d_rope, cfg.d_v, cfg.dtype, cfg.rope_base)
    B, L, S = args.loop_batch, args.layers, args.loop_context
    layers = random_layers(lc, L, cfg.d_model, cfg.q_lora, dev, seed=7)
    stack = DecodeStack(lc, layers, batch=B, capacity=S + args.warmup + args.steps + 2)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    h_prefix = torch.randn((B, S, cfg.d_model), generator=gen, device=dev).to(torch.bfloat16)
    t0 = time.time()
    stack.forward(h_prefix)
    torch.cuda.synchronize()
    prefill_s = time.time() - t0
    del h_prefix
    g = stack.capture_decode()
    g.h_in.copy_(torch.randn((B, 1, cfg.d_model), generator=gen, device=dev).to(torch.bfloat16))
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ctx0 = stack.length
    start.record(stream)
    for _ in range(args.steps):
        g.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_token = start.elapsed_time(stop) / args.steps
    esz = 2
    w_bytes = sum(t.numel() * esz for t in layers[0].values()) * L
    keys = B * (ctx0 + 1 + args.steps / 2.0)               # mean keys per sequence over the timed tokens
    cache_bytes = keys * cfg.row * esz * L
    moved = w_bytes + cache_bytes
    gbs = moved / (ms_token * 1e-3) / 1e9
    print(json.dumps({
        "metric": "MLA decode loop: per-token latency through a stack of full attention layers",
        "value": round(B / (ms_token * 1e-3), 2), "unit": "tokens/s", "ms_per_token": round(ms_token, 4),
        "steps": args.steps, "warmup": args.warmup, "launch": "hip_graph", "dtype": "bf16",
        "data": "synthetic (seeded device N(0,1/fan_in) weights and N(0,1) hidden states)",
        "config": {"workload": "v3_decode_loop", "layers": L, "batch": B, "context_tokens": ctx0,
                   "d_model": cfg.d_model, "q_lora": cfg.q_lora, "heads": cfg.n_heads},
        "bytes_per_token": {"weights": w_bytes, "cache": int(cache_bytes)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)},
        "prefill_s": round(prefill_s, 3),
    }), flush=True)


def merged_wo_check(args):
    """The output side of one decode token (batch 1, DeepSeek-V3 shape), two ways:
    separate — mla_out_proj with W_O: o_i = W_UV,i z_i, then u = W_O concat(o) (16.8 + 235 MB of weights);
    merged  — u = (W_O W_UV) z with the pre-multiplied [7168 x 65536] matrix (940 MB), run through the
              library's linear kernel (mla_project_q on a 56-head layer description whose W_UQ is that
              matrix: one output row of 7168 values from 65536 inputs).
    Each weight set is replicated so every timed call reads its weights from HBM."""
    import torch

    import mla_decode_decoupled_amd as mla

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16
    H, dv, dc, dm = 128, 128, 512, 7168
    lc = mla.make_config(H, 128, dc, 64, dv, "bf16", 10000.0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    reps = 4
    z = torch.randn((1, H, dc), generator=gen, device=dev)
    zb = z.to(bf).view(1, H * dc)
    sep = [((torch.randn((H, dv, dc), generator=gen, device=dev) / dc ** 0.5).to(bf),
            (torch.randn((dm, H * dv), generator=gen, device=dev) / (H * dv) ** 0.5).to(bf)) for _ in range(reps)]
    merged = [(torch.randn((dm, H * dc), generator=gen, device=dev) / (H * dc) ** 0.5).to(bf) for _ in range(reps)]
    o = torch.empty((1, H, dv), dtype=bf, device=dev)
    u = torch.empty((1, dm), dtype=bf, device=dev)
    lm = mla.make_config(dm // 128, 128, dc, 0, 128, "bf16", 10000.0)   # W_UQ rows = 56 * 128 = 7168
    qn = torch.empty((1, dm // 128, 128), dtype=bf, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn, n):
        for i in range(reps):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i % reps)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    t_sep = timed(lambda i: mla.mla_out_proj(lc, z, sep[i][0], o, w_o=sep[i][1], u=u), args.steps)
    t_mer = timed(lambda i: mla.mla_project_q(lm, zb, merged[i], None, qn, None), args.steps)
    print(json.dumps({"metric": "output side of one batch-1 decode token", "unit": "us",
                      "separate_us": round(t_sep, 2), "separate_weight_bytes": (H * dv * dc + dm * H * dv) * 2,
                      "merged_us": round(t_mer, 2), "merged_weight_bytes": dm * H * dc * 2,
                      "steps": args.steps}), flush=True)


def cpu_baseline(cfg, c_host, k_host, qn_host, qr_host, wuk_host, wuv_host, lens, budget_s):
    """The fp64 oracle on the host cores over a bounded sample of the same workload."""
    import numpy as np

    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    H, n_q = cfg.n_heads, cfg.n_q
    # sample: sequence 0, its query rows, heads taken in order until the time budget is used
    b = 0
    qn = qn_host[b * n_q:(b + 1) * n_q]
    qr = qr_host[b * n_q:(b + 1) * n_q]
    rows = list(range(n_q)) if n_q <= 4 else [0, n_q // 2, n_q - 1]
    t0 = time.perf_counter()
    heads_done = 0   # head evaluations, cycling over the heads in groups of 8 until the budget is used
    while (time.perf_counter() - t0) < budget_s:
        h0 = heads_done % H
        hs = list(range(h0, min(H, h0 + 8)))
        O.explicit_attention(c_host[b], k_host[b], qn, qr, wuk_host, wuv_host, scale=cfg.softmax_scale,
                             base=cfg.rope_base, heads=hs, rows=rows)
        heads_done += len(hs)
    el = time.perf_counter() - t0
    # scale the sample (heads_done head evaluations of len(rows) query rows) to whole query tokens
    tokens = (heads_done / H) * len(rows)
    return {"value": round(tokens / el, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"sequence 0 ({int(lens[0])} keys), {len(rows)} query row(s), {heads_done} head evaluations "
                      f"({heads_done / H:.1f} x all {H} heads) in {el:.1f} s of the fp64 non-absorbed oracle; "
                      f"tokens/s = whole-token equivalents / s"}


if __name__ == "__main__":
    main()
