#!/usr/bin/env python3
"""Benchmark of absorbed-MLA decode with decoupled RoPE on one MI355X.

Headline: one step = one pass of the whole hot path over one batch: the append of
the new tokens, the query absorption, the latent attention with its split-K merge,
and the W_UV projection, as one mla_decode_step call (or, with --single-calls, as
mla_rope_append, mla_absorb_q, mla_decode_attn and mla_out_proj). The default
workload is the DeepSeek-V3-shaped decode step (batch 1, 128 heads, 512-dim
latent, 64-dim position part, 4096 cached tokens + 1 new, bf16). Inputs are
seeded synthetic data of that shape and are resident in HBM before timing starts.

Timing protocol (independent of --steps): the K = --steps timed steps are
captured once as one HIP graph; step i reads input copy i mod C, with C copies of
the cache, weights and queries (C = min(K, enough for 1 GiB, four times the 256 MB
last-level cache)), so the bytes come from HBM. The graph is replayed once
untimed, then --reps times, each replay bracketed by synchronisations; ms_per_step
is the median replay time / K, with p10 and p90 over the replays. The step
launched eagerly from Python (one replay's worth of steps) is reported too.

Per-call timing: the single calls run again, each bracketed by HIP events on the
launch stream with a spin kernel ahead, so an interval is GPU time only; the mean
of mla_decode_attn's intervals is the roofline's launch duration.

Per-workload rooflines: unless --no-per-config, the attention call is timed the
same way on the four DeepSeek-shaped workloads (batch 1 at 4K keys; ragged batch
64; batch 4 at 128K keys; chunked prefill of 2 x 2048 rows), and the chunked
prefill also through mla_prefill_explicit, each with its algorithmic bytes and
flops, the fraction of the binding roofline and the HBM traffic recorded by the
committed counter summary for the current attention sources.

Prints one JSON line with throughput, the roofline object of the dominant call
and the fp64 CPU oracle timed on a bounded sample of the same workload.
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
COLD_BYTES = 1 << 30           # working set of the rotated copies: 4x the 256 MB last-level cache


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=11, help="timed replays of the K-step graph (median reported)")
    ap.add_argument("--config", type=int, default=1, help="workload id (1 = V3 decode, batch 1, S=4096)")
    ap.add_argument("--n-splits", type=int, default=0, help="split-K chunks per sequence (0 = library choice)")
    ap.add_argument("--hot", action="store_true", help="reuse one copy of every input (cache-hot numbers)")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0 = enough for 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget for the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true", help="skip the per-workload attention rooflines")
    ap.add_argument("--per-configs", default="1,2,3,4", help="workloads of the per-workload rooflines")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps launched from Python instead of replaying the captured graph")
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--single-calls", action="store_true",
                    help="time the step as the four single calls instead of one mla_decode_step")
    ap.add_argument("--explicit", action="store_true",
                    help="many-row workloads: the step is mla_rope_append + mla_prefill_explicit (the non-absorbed "
                         "form) instead of absorb + latent attention + W_UV")
    ap.add_argument("--attn-only", action="store_true",
                    help="run only the attention call of --config (eagerly, --steps calls over cold copies): the "
                         "command the counter summaries are taken with")
    ap.add_argument("--merged-wo-check", action="store_true",
                    help="time the output side at batch 1 both ways: W_UV per head then W_O (the library's "
                         "path) against one pre-merged [d_model x H*d_latent] matrix W_O W_UV applied to z")
    ap.add_argument("--a16-check", action="store_true",
                    help="time the query side at batch 1 both ways: W_UQ (+ W_QR) then the W_UK absorption "
                         "(the library's path) against one pre-merged [H*d_latent x q_lora] matrix W_UK^T W_UQ")
    ap.add_argument("--prefill-crossover", action="store_true",
                    help="time the absorbed and the explicit attention for a range of query rows per sequence "
                         "(2 sequences, 4096 keys) to place the switch between them")
    ap.add_argument("--decode-loop", action="store_true",
                    help="instead of the single step: time token-by-token decode through a stack of full MLA "
                         "layers (h -> projections -> attention -> W_O) replayed as one HIP graph per token")
    ap.add_argument("--layers", type=int, default=61, help="--decode-loop: layers in the stack")
    ap.add_argument("--loop-context", type=int, default=4096, help="--decode-loop: tokens prefilled per sequence")
    ap.add_argument("--loop-batch", type=int, default=1, help="--decode-loop: sequences decoded together")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the step: time a plain 1 GiB device copy (the reference kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="measure chip-wide bf16 MFMA issue (1 and 2 waves per SIMD) and the clock it ran at")
    ap.add_argument("--lds-ceiling", action="store_true",
                    help="measure LDS read throughput per CU for ds_read_b128 and ds_read_b64_tr_b16")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="per-phase time of the attention kernels' workgroups (diagnostic build libmla_stamps.so)")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="measure read-only HBM streaming: vector loads, and the attention kernel's LDS tile ring")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------------------
# recorded HBM traffic (FETCH_SIZE / WRITE_SIZE, scaled by the plain-copy calibration)

COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_traffic_counters.md")
TRAFFIC_SOURCES = [os.path.join(ROOT, "mla_decode_decoupled_amd", "csrc", f)
                   for f in ("api.hip", "generic.hip", "decode_fast.hip", "prefill_explicit.hip", "linear.hip")]


def sources_sha(paths=None) -> str:
    """Hash of the code of the sources that decide what the attention kernels read and write: their
    text with the comments, trailing blanks and empty lines taken out, so that a comment edit keeps the
    records valid and any change to the code does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES if paths is None else paths:
        with open(f, encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        lines = (re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines())
        h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, call: str, n_splits: int, cold: bool):
    """HBM bytes per call of `call` on `workload`, as recorded by the committed counter summary, or None
    when there is no record for it, the inputs were cache-hot, or the kernels changed since."""
    try:
        text = open(COUNTERS_FILE).read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        recs = json.loads(block)["records"]
    except (OSError, IndexError, ValueError, KeyError):
        return None
    if not cold:
        return None
    sha = sources_sha()
    for rec in recs:
        if (rec.get("workload") == workload and rec.get("call") == call and rec.get("n_splits") == n_splits
                and rec.get("source_sha") == sha):
            return rec.get("traffic_bytes_per_call")
    return None


# ---------------------------------------------------------------------------------------------------
# small helpers

def _pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def _stats(ms_list):
    import numpy as np
    a = np.asarray(ms_list, dtype=np.float64)
    return {"mean": round(float(a.mean()), 6), "median": round(float(np.median(a)), 6),
            "p10": round(_pct(a, 10), 6), "p90": round(_pct(a, 90), 6), "n": int(a.size)}


def _device():
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return dev


def roofline_of(bytes_, flops, ms, traffic=None, kernel="mla_decode_attn"):
    """Roofline object of one call: the binding bound is the larger of bytes / 8 TB/s and
    flops / 2.5 PFLOP/s; `achieved` is the algorithmic amount of that bound per measured second."""
    t_bw, t_mf = bytes_ / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
    s = ms * 1e-3
    if t_bw >= t_mf:
        achieved, peak, unit, bound = bytes_ / s / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = flops / s / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    return {"kernel": kernel, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "algorithmic_bytes_per_launch": int(bytes_),
            "algorithmic_flops_per_launch": int(flops), "avg_launch_ms": round(ms, 6),
            "gbs": round(bytes_ / s / 1e9, 2), "tflops": round(flops / s / 1e12, 2)}


class Workload:
    """Seeded inputs of one workload on the device, C cold copies of (cache, W_UK, W_UV, q_nope, q_rope)."""

    def __init__(self, cid: int, dev, n_copies_max: int, hot: bool, copies: int = 0, weights: bool = True):
        import numpy as np
        import torch

        import mla_decode_decoupled_amd as mla
        from mla_workloads import get_config
        from mla_workloads import generate as G

        cfg = get_config(cid)
        self.cfg = cfg
        self.lc = mla.make_config(cfg.n_heads, cfg.d_nope, cfg.d_latent, cfg.d_rope, cfg.d_v, cfg.dtype,
                                  cfg.rope_base)
        dt = mla.storage_dtype(self.lc)
        self.dt = dt
        self.esz = 2 if cfg.dtype == "bf16" else 4
        B, n_q, H, row = cfg.batch, cfg.n_q, cfg.n_heads, cfg.row
        lens = G.seq_lens(cfg)
        self.lens = lens
        self.B, self.n_q, self.H, self.row, self.R = B, n_q, H, row, B * n_q
        self.max_len = int(lens.max())
        self.c_host = [G.cache_latent(cfg, b, int(lens[b])) for b in range(B)]
        self.k_host = [G.cache_rope_pre(cfg, b, int(lens[b])) for b in range(B)]
        self.qn_host = np.stack([G.query_nope(cfg, b) for b in range(B)]).reshape(self.R, H, cfg.d_nope)
        self.qr_host = np.stack([G.query_rope_pre(cfg, b) for b in range(B)]).reshape(self.R, H, cfg.d_rope)
        self.wuk_host, self.wuv_host = G.weight_uk(cfg), G.weight_uv(cfg)
        up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)  # noqa: E731
        offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        self.seq_off = torch.from_numpy(offs).to(dev)
        self.seq_len = torch.from_numpy(lens.astype(np.int32)).to(dev)
        self.len_before = torch.from_numpy((lens - n_q).astype(np.int32)).to(dev)
        self.q_pos = torch.from_numpy(
            np.concatenate([np.arange(int(l) - n_q, int(l)) for l in lens]).astype(np.int32)).to(dev)
        self.c_new = up(np.stack([self.c_host[b][int(lens[b]) - n_q:] for b in range(B)]))
        self.k_new = up(np.stack([self.k_host[b][int(lens[b]) - n_q:] for b in range(B)]))
        # one copy: the cache history appended by the library itself, weights, queries
        cache0 = torch.empty((int(lens.sum()), row), dtype=dt, device=dev)
        for b in range(B):
            h = int(lens[b]) - n_q
            if h > 0:
                mla.mla_rope_append(self.lc, up(self.c_host[b][None, :h]), up(self.k_host[b][None, :h]), cache0,
                                    self.seq_off[b:b + 1], torch.zeros(1, dtype=torch.int32, device=dev))
        # the new tokens too, so that the attention-only calls see every key (the step rewrites them)
        mla.mla_rope_append(self.lc, self.c_new, self.k_new, cache0, self.seq_off, self.len_before)
        first = (cache0, up(self.wuk_host), up(self.wuv_host), up(self.qn_host), up(self.qr_host))
        self.per_copy = sum(t.numel() for t in first) * self.esz
        if hot:
            n = 1
        else:
            n = copies or max(1, min(64, math.ceil(COLD_BYTES / self.per_copy)))
            n = max(1, min(n, n_copies_max))
        self.copies = [first] + [tuple(t.clone() for t in first) for _ in range(n - 1)]
        self.n_copies = n
        self.hot = hot
        # outputs and workspaces, shared by all copies
        self.q_packed = torch.empty((self.R, H, row), dtype=dt, device=dev)
        self.z = torch.empty((B, n_q, H, cfg.d_latent), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev)
        self.o = torch.empty((self.R, H, cfg.d_v), dtype=dt, device=dev)
        self.dev = dev
        torch.cuda.synchronize()

    # algorithmic work of the attention call (absorbed) and of the explicit prefill
    def vis_pairs(self):
        n_q = self.n_q
        if n_q == 1:
            return int(self.lens.sum())
        return int(sum(n_q * (int(l) - n_q) + n_q * (n_q + 1) // 2 for l in self.lens))

    def attn_bytes_flops(self):
        cfg, H, R, esz = self.cfg, self.H, self.R, self.esz
        keys = int(self.lens.sum())
        b = keys * self.row * esz + R * H * self.row * esz + R * H * cfg.d_latent * 4 + R * H * 4
        f = 2 * H * (self.row + cfg.d_latent) * self.vis_pairs()
        return b, f

    def explicit_bytes_flops(self):
        cfg, H, R, esz = self.cfg, self.H, self.R, self.esz
        keys = int(self.lens.sum())
        f = (2 * H * (cfg.d_nope + cfg.d_rope + cfg.d_v) * self.vis_pairs()
             + 2 * keys * cfg.d_latent * H * (cfg.d_nope + cfg.d_v))
        b = (keys * self.row * esz + 2 * keys * H * (cfg.d_nope + cfg.d_v) * esz
             + 2 * H * cfg.d_nope * cfg.d_latent * esz
             + R * H * (cfg.d_nope + cfg.d_rope) * esz + R * H * cfg.d_v * esz + R * H * 4)
        return b, f


def _events_time(stream, fn, n, spin=True):
    """Per-call GPU intervals (ms): fn(i) bracketed by events; a spin kernel ahead of each call keeps
    the GPU busy while Python enqueues, so an interval holds only the call's own GPU time."""
    import torch
    marks = []
    for i in range(n):
        if spin:
            torch.cuda._sleep(200_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn(i)
        b.record(stream)
        marks.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in marks]


def _graph_reps(stream, fn, k, reps):
    """Capture k calls fn(0..k-1) as one HIP graph, replay it once untimed, then `reps` times, each
    replay between synchronisations; returns the per-replay ms / k."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(k):
            fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / k)
    del g
    return out


# ---------------------------------------------------------------------------------------------------
# per-workload attention rooflines

def attn_config_entry(cid: int, dev, steps: int, warmup: int, hot: bool, verbose: bool):
    """mla_decode_attn (and, for many query rows, mla_prefill_explicit) on one workload: per-call GPU
    time over `steps` calls that rotate over cold copies, with the roofline of the call."""
    import torch

    import mla_decode_decoupled_amd as mla

    t0 = time.time()
    W = Workload(cid, dev, steps, hot)
    cfg, lc = W.cfg, W.lc
    B, n_q, H = W.B, W.n_q, W.H
    n_splits = cfg.n_splits
    stream = torch.cuda.current_stream(dev)
    ws = torch.empty(max(16, mla.mla_decode_attn_workspace_size(lc, B, n_q, W.max_len, n_splits)), dtype=torch.uint8,
                     device=dev)
    # q_packed of every copy: absorbed once from that copy's queries and W_UK
    qps = []
    for (_, wuk, _, qn, qr) in W.copies:
        qp = torch.empty_like(W.q_packed)
        mla.mla_absorb_q(lc, qn, qr, W.q_pos, wuk, qp)
        qps.append(qp.view(B, n_q, H, W.row))
    torch.cuda.synchronize()

    def attn(i):
        c = i % W.n_copies
        mla.mla_decode_attn(lc, qps[c], W.copies[c][0], W.seq_off, W.seq_len, W.max_len, W.z, W.lse,
                            n_splits=n_splits, workspace=ws)

    for i in range(warmup):
        attn(i)
    torch.cuda.synchronize()
    per_call = _events_time(stream, attn, steps)
    st = _stats(per_call)
    b, f = W.attn_bytes_flops()
    entry = {"workload": cfg.name, "call": "mla_decode_attn", "batch": B, "n_q": n_q,
             "keys": int(W.lens.sum()), "n_splits": n_splits, "cold_copies": W.n_copies,
             "call_ms": st,
             "roofline": roofline_of(b, f, st["mean"], recorded_traffic(cfg.name, "mla_decode_attn", n_splits,
                                                                        not hot))}
    entry["roofline"]["frac_median"] = round(entry["roofline"]["frac"] * st["mean"] / st["median"], 4)
    del qps, ws
    if n_q > 1:
        # chunked prefill: the non-absorbed form, rebuilt keys and values, o written directly
        wsx = torch.empty(max(16, mla.mla_prefill_explicit_workspace_size(lc, B, n_q, W.max_len)),
                          dtype=torch.uint8, device=dev)

        def expl(i):
            c = W.copies[i % W.n_copies]
            mla.mla_prefill_explicit(lc, c[3].view(B, n_q, H, cfg.d_nope), c[4].view(B, n_q, H, cfg.d_rope), c[0],
                                     W.seq_off, W.seq_len, W.max_len, c[1], c[2], W.o.view(B, n_q, H, cfg.d_v),
                                     lse=W.lse, workspace=wsx)

        for i in range(warmup):
            expl(i)
        torch.cuda.synchronize()
        sx = _stats(_events_time(stream, expl, steps))
        bx, fx = W.explicit_bytes_flops()
        entry["explicit"] = {"call": "mla_prefill_explicit", "call_ms": sx,
                             "roofline": roofline_of(bx, fx, sx["mean"],
                                                     recorded_traffic(cfg.name, "mla_prefill_explicit", 0, not hot),
                                                     kernel="mla_prefill_explicit"),
                             "absorbed_step_flops": int(f + 2 * 2 * W.R * H * cfg.d_nope * cfg.d_latent),
                             "prefers_explicit": bool(mla.mla_prefill_prefers_explicit(lc, B, n_q, W.max_len))}
        del wsx
    entry["setup_s"] = round(time.time() - t0, 1)
    del W
    torch.cuda.empty_cache()
    if verbose:
        print(json.dumps(entry), file=sys.stderr, flush=True)
    return entry


def attn_only(args):
    """--attn-only: the attention call of one workload, eagerly, over cold copies (counter runs)."""
    import torch

    import mla_decode_decoupled_amd as mla

    dev = _device()
    W = Workload(args.config, dev, args.steps, args.hot, args.copies)
    cfg, lc = W.cfg, W.lc
    B, n_q, H = W.B, W.n_q, W.H
    n_splits = args.n_splits or cfg.n_splits
    if args.explicit:
        wsx = torch.empty(max(16, mla.mla_prefill_explicit_workspace_size(lc, B, n_q, W.max_len)),
                          dtype=torch.uint8, device=dev)
        for i in range(args.warmup + args.steps):
            c = W.copies[i % W.n_copies]
            mla.mla_prefill_explicit(lc, c[3].view(B, n_q, H, cfg.d_nope), c[4].view(B, n_q, H, cfg.d_rope), c[0],
                                     W.seq_off, W.seq_len, W.max_len, c[1], c[2], W.o.view(B, n_q, H, cfg.d_v),
                                     lse=W.lse, workspace=wsx)
    else:
        ws = torch.empty(max(16, mla.mla_decode_attn_workspace_size(lc, B, n_q, W.max_len, n_splits)),
                         dtype=torch.uint8, device=dev)
        qps = []
        for (_, wuk, _, qn, qr) in W.copies:
            qp = torch.empty_like(W.q_packed)
            mla.mla_absorb_q(lc, qn, qr, W.q_pos, wuk, qp)
            qps.append(qp.view(B, n_q, H, W.row))
        for i in range(args.warmup + args.steps):
            c = i % W.n_copies
            mla.mla_decode_attn(lc, qps[c], W.copies[c][0], W.seq_off, W.seq_len, W.max_len, W.z, W.lse,
                                n_splits=n_splits, workspace=ws)
    torch.cuda.synchronize()
    print(json.dumps({"attn_only": cfg.name, "calls": args.warmup + args.steps, "copies": W.n_copies,
                      "explicit": bool(args.explicit), "n_splits": n_splits, "source_sha": sources_sha()}),
          flush=True)


def stamp_summary(st):
    """Per-workgroup phases of one launch from the stamp array (uint64 [workgroups, 16], see
    include/mla_stamps.h): medians and spreads in µs, each workgroup's cycles at its own clock."""
    import numpy as np

    act = st[(st[:, 5] != 0) & (st[:, 0] != 0) & ((st[:, 13] == 1) | (st[:, 13] == 2))]
    if len(act) == 0:
        return None
    kern = int(act[0, 13])
    real_us = (act[:, 9].astype(np.float64) - act[:, 8]) / 100.0           # 100 MHz counter
    cyc = act[:, 5].astype(np.float64) - act[:, 0]
    ghz = cyc / (real_us * 1e3)
    phases = {"chunk_plan": (0, 1), "queries_to_registers": (1, 2), "first_tiles_issued": (2, 3),
              "tile_loop": (3, 4), "stores_to_exit": (4, 5), "workgroup_total": (0, 5)}
    if kern == 2:
        phases = {"chunk_plan": (0, 1), "queries_and_first_tiles_landed": (1, 3), "tile_loop": (3, 4),
                  "stores_to_exit": (4, 5), "workgroup_total": (0, 5)}
    out = {"kernel": "decode_attn_fast" if kern == 1 else "decode_attn_hsplit", "workgroups": int(len(act)),
           "clock_ghz_median": round(float(np.median(ghz)), 3)}
    for name, (a, b) in phases.items():
        us = (act[:, b].astype(np.float64) - act[:, a]) / (ghz * 1e3)
        out[name + "_us"] = {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
                             "p90": round(float(np.percentile(us, 90)), 2)}
    tiles = act[:, 10].astype(np.float64)
    loop_cyc = act[:, 4].astype(np.float64) - act[:, 3]
    per_tile = loop_cyc[tiles > 0] / tiles[tiles > 0]
    out["tiles_per_workgroup"] = {"median": float(np.median(tiles)), "min": int(tiles.min()), "max": int(tiles.max())}
    out["cycles_per_tile_median"] = round(float(np.median(per_tile)), 1)
    r0, r1 = act[:, 8].astype(np.float64), act[:, 9].astype(np.float64)
    out["start_spread_us"] = round(float(r0.max() - r0.min()) / 100.0, 2)
    out["end_spread_us"] = round(float(r1.max() - r1.min()) / 100.0, 2)
    out["first_start_to_last_end_us"] = round(float(r1.max() - r0.min()) / 100.0, 2)
    return out


def phase_stamps(args):
    """--phase-stamps: mla_decode_attn on each workload through the phase-stamp build of the library
    (libmla_stamps.so: the same kernels with per-workgroup clock stamps, include/mla_stamps.h), and
    where the workgroups' time goes: chunk plan, query staging, first tiles, the tile loop (and its
    cycles per tile), the output stores, and the spread of the workgroups' start and end times."""
    import ctypes

    import numpy as np

    path = os.path.join(ROOT, "mla_decode_decoupled_amd", "libmla_stamps.so")
    if "mla_decode_decoupled_amd" in sys.modules:
        raise SystemExit("--phase-stamps must load the stamp build before the library")
    os.environ["MLA_LIB_PATH"] = path
    import torch

    import mla_decode_decoupled_amd as mla

    lib = ctypes.CDLL(path)
    lib.mla_phase_stamps_bytes.restype = ctypes.c_size_t
    lib.mla_phase_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    nbytes = lib.mla_phase_stamps_bytes()
    host = np.zeros(nbytes // 8, dtype=np.uint64)
    dev = _device()
    res = []
    for cid in [int(x) for x in args.per_configs.split(",") if x.strip()]:
        W = Workload(cid, dev, max(2, args.steps), args.hot)
        cfg, lc = W.cfg, W.lc
        B, n_q, H = W.B, W.n_q, W.H
        ws = torch.empty(max(16, mla.mla_decode_attn_workspace_size(lc, B, n_q, W.max_len, cfg.n_splits)),
                         dtype=torch.uint8, device=dev)
        qps = []
        for (_, wuk, _, qn, qr) in W.copies:
            qp = torch.empty_like(W.q_packed)
            mla.mla_absorb_q(lc, qn, qr, W.q_pos, wuk, qp)
            qps.append(qp.view(B, n_q, H, W.row))

        def attn(i):
            c = i % W.n_copies
            mla.mla_decode_attn(lc, qps[c], W.copies[c][0], W.seq_off, W.seq_len, W.max_len, W.z, W.lse,
                                n_splits=cfg.n_splits, workspace=ws)

        for i in range(max(1, args.warmup)):
            attn(i)
        torch.cuda.synchronize()
        runs = []
        for i in range(args.steps):
            if lib.mla_phase_stamps_clear() != 0:
                raise RuntimeError("mla_phase_stamps_clear failed")
            attn(i)
            torch.cuda.synchronize()
            if lib.mla_phase_stamps_read(host.ctypes.data, nbytes) != 0:
                raise RuntimeError("mla_phase_stamps_read failed")
            summ = stamp_summary(host.reshape(-1, 16))
            if summ is not None:
                runs.append(summ)
        # the median call by its first-start-to-last-end span
        runs.sort(key=lambda r: r["first_start_to_last_end_us"])
        entry = {"workload": cfg.name, "call": "mla_decode_attn", "calls": len(runs),
                 "median_call": runs[len(runs) // 2] if runs else None,
                 "span_us_all_calls": [r["first_start_to_last_end_us"] for r in runs]}
        res.append(entry)
        del qps, ws, W
        torch.cuda.empty_cache()
    print(json.dumps({"phase_stamps": res, "library": "libmla_stamps.so",
                      "note": "each call's stamps read back after it; one call per cold copy"}), flush=True)


# ---------------------------------------------------------------------------------------------------
# the headline step

def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    modes = {"copy_calibration": copy_calibration, "decode_loop": decode_loop, "merged_wo_check": merged_wo_check,
             "a16_check": a16_check, "mfma_peak": mfma_peak, "stream_ceiling": stream_ceiling,
             "lds_ceiling": lds_ceiling,
             "attn_only": attn_only, "prefill_crossover": prefill_crossover, "phase_stamps": phase_stamps}
    for name, fn in modes.items():
        if getattr(args, name):
            fn(args)
            return

    import numpy as np
    import torch

    import mla_decode_decoupled_amd as mla

    dev = _device()
    t_setup = time.time()
    K = args.steps
    W = Workload(args.config, dev, K, args.hot, args.copies)
    cfg, lc = W.cfg, W.lc
    B, n_q, H, R = W.B, W.n_q, W.H, W.R
    n_splits = args.n_splits or cfg.n_splits
    if args.explicit:
        ws = torch.empty(max(16, mla.mla_prefill_explicit_workspace_size(lc, B, n_q, W.max_len)), dtype=torch.uint8,
                         device=dev)
        if ws.numel() == 16:
            raise SystemExit("--explicit needs the bf16 DeepSeek head shape and n_q <= keys")
    else:
        ws = torch.empty(max(16, mla.mla_decode_attn_workspace_size(lc, B, n_q, W.max_len, n_splits)),
                         dtype=torch.uint8, device=dev)
    ws_step = torch.empty(max(16, mla.mla_decode_step_workspace_size(lc, B, n_q, W.max_len, n_splits)),
                          dtype=torch.uint8, device=dev)
    fused = not args.explicit and not args.single_calls
    stream = torch.cuda.current_stream(dev)
    setup_s = time.time() - t_setup

    def single_calls(i, marks=None):
        cache, wuk, wuv, qn, qr = W.copies[i % W.n_copies]
        rec = (lambda j: marks[j].record(stream)) if marks is not None else (lambda j: None)
        rec(0)
        mla.mla_rope_append(lc, W.c_new, W.k_new, cache, W.seq_off, W.len_before)
        rec(1)
        if args.explicit:
            rec(2)
            mla.mla_prefill_explicit(lc, qn.view(B, n_q, H, cfg.d_nope), qr.view(B, n_q, H, cfg.d_rope), cache,
                                     W.seq_off, W.seq_len, W.max_len, wuk, wuv, W.o.view(B, n_q, H, cfg.d_v),
                                     lse=W.lse, workspace=ws)
            rec(3)
            rec(4)
            return
        mla.mla_absorb_q(lc, qn, qr, W.q_pos, wuk, W.q_packed)
        rec(2)
        mla.mla_decode_attn(lc, W.q_packed.view(B, n_q, H, W.row), cache, W.seq_off, W.seq_len, W.max_len, W.z,
                            W.lse, n_splits=n_splits, workspace=ws)
        rec(3)
        mla.mla_out_proj(lc, W.z.view(R, H, cfg.d_latent), wuv, W.o)
        rec(4)

    def step(i):
        if not fused:
            single_calls(i)
            return
        cache, wuk, wuv, qn, qr = W.copies[i % W.n_copies]
        mla.mla_decode_step(lc, W.c_new, W.k_new, qn, qr, wuk, wuv, cache, W.seq_off, W.seq_len, W.max_len,
                            W.q_packed, W.z, W.o, lse=W.lse, n_splits=n_splits, workspace=ws_step)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # eager: K steps launched from Python (bound by launch overhead at batch 1)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(K):
        step(i)
    b.record(stream)
    torch.cuda.synchronize()
    ms_step_eager = a.elapsed_time(b) / K

    # the headline: the K steps as one captured graph, replayed --reps times
    if args.eager:
        reps_ms = []
        for _ in range(args.reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for i in range(K):
                step(i)
            b.record(stream)
            torch.cuda.synchronize()
            reps_ms.append(a.elapsed_time(b) / K)
    else:
        reps_ms = _graph_reps(stream, step, K, args.reps)
    ms_step = float(np.median(reps_ms))

    # per-call pass: each call between events, GPU time only (the single calls' kernels are
    # launched a few times first: a kernel's first launch also loads its code)
    for i in range(max(2, args.warmup)):
        single_calls(i)
    torch.cuda.synchronize()
    ev = {k: [] for k in ("append", "absorb", "attn", "proj")}
    for i in range(K):
        torch.cuda._sleep(200_000)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        single_calls(i, marks)
        for j, k in enumerate(("append", "absorb", "attn", "proj")):
            ev[k].append((marks[j], marks[j + 1]))
    torch.cuda.synchronize()
    per_call = {k: _stats([x.elapsed_time(y) for x, y in v]) for k, v in ev.items()}

    # algorithmic work of each call
    esz = W.esz
    if args.explicit:
        attn_b, attn_f = W.explicit_bytes_flops()
    else:
        attn_b, attn_f = W.attn_bytes_flops()
    kernel_bytes = {
        "append": R * (cfg.d_latent + cfg.d_rope) * esz + R * W.row * esz,
        "absorb": H * cfg.d_nope * cfg.d_latent * esz + R * H * (cfg.d_nope + cfg.d_rope) * esz + R * H * W.row * esz,
        "attn": attn_b,
        "proj": H * cfg.d_v * cfg.d_latent * esz + R * H * cfg.d_latent * 4 + R * H * cfg.d_v * esz,
    }
    call_name = {"attn": "mla_prefill_explicit" if args.explicit else "mla_decode_attn", "absorb": "mla_absorb_q",
                 "proj": "mla_out_proj", "append": "mla_rope_append"}
    dominant = max(per_call, key=lambda k: per_call[k]["mean"])
    if dominant == "attn":
        roof = roofline_of(attn_b, attn_f, per_call["attn"]["mean"],
                           recorded_traffic(cfg.name, call_name["attn"], n_splits, not args.hot))
    else:
        roof = roofline_of(kernel_bytes[dominant], 0, per_call[dominant]["mean"], None, call_name[dominant])
    roof["kernel"] = call_name[dominant]
    roof["timing"] = ("mean of HIP-event intervals around each call on its launch stream, "
                      f"{K} calls over {W.n_copies} cold copies")
    tokens_per_s = R / (ms_step * 1e-3)

    # per-workload attention rooflines (the metric spans 4K to 128K keys)
    per_config = None
    if not args.no_per_config:
        # the headline's device copies are no longer needed; its host inputs serve the CPU baseline
        W.copies = W.copies[:1]
        del ws, ws_step
        torch.cuda.empty_cache()
        per_config = []
        for cid in [int(x) for x in args.per_configs.split(",") if x.strip()]:
            per_config.append(attn_config_entry(cid, dev, K, max(1, args.warmup // 2), args.hot, args.verbose))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(W, args.cpu_seconds, explicit=args.explicit)

    out = {
        "metric": "MLA decode tokens/s + achieved HBM GB/s (H=128, d_c=512, S=4K-128K)",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "ms_per_step_p10": round(_pct(reps_ms, 10), 6),
        "ms_per_step_p90": round(_pct(reps_ms, 90), 6),
        "timed_reps": len(reps_ms),
        "ms_per_step_eager": round(ms_step_eager, 6),
        "launch": "eager" if args.eager else "hip_graph",
        "step_call": ("mla_rope_append + mla_prefill_explicit" if args.explicit
                      else "mla_decode_step" if fused else "four single calls"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) inputs, N(0,1/fan_in) weights, RMS-normalised latent)",
        "config": {"workload": cfg.name + ("_explicit" if args.explicit else ""), "batch": B, "n_q": n_q,
                   "heads": H, "d_latent": cfg.d_latent, "d_rope": cfg.d_rope, "d_nope": cfg.d_nope, "d_v": cfg.d_v,
                   "seq_len_keys": (int(W.max_len) if len(set(W.lens.tolist())) == 1
                                    else [int(W.lens.min()), int(W.lens.max())]),
                   "n_splits": n_splits, "cold_copies": W.n_copies, "parallelism": "single GPU"},
        "roofline": roof,
        "calls_ms": per_call,
        "per_config": per_config,
        "cpu_baseline": cpu,
    }
    if args.verbose:
        print(f"setup {setup_s:.1f}s, copies {W.n_copies} x {W.per_copy / 1e6:.1f} MB", file=sys.stderr)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores

def cpu_baseline(W, budget_s, explicit=False):
    """The fp64 non-absorbed oracle on the host cores over a bounded sample of the same workload:
    all cores of this process's affinity mask (BLAS threads pinned to that count), plus one thread.
    The oracle's outputs for the heads it evaluates are also compared with the GPU's result of the
    last timed call on the same inputs (z, or o for the explicit path): the run's own parity check."""
    import numpy as np

    import oracle as O
    from mla_workloads import get_config
    from mla_workloads import generate as G

    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    cfg, H, n_q = W.cfg, W.H, W.n_q
    b = 0
    qn = W.qn_host[b * n_q:(b + 1) * n_q]
    qr = W.qr_host[b * n_q:(b + 1) * n_q]
    rows = list(range(n_q)) if n_q <= 4 else [0, n_q // 2, n_q - 1]
    # the GPU's result for sequence 0's sampled rows (every copy holds the same inputs)
    key = "o" if explicit else "z"
    gpu = (W.o[b * n_q:(b + 1) * n_q] if explicit else W.z[b]).float().cpu().numpy()[rows]
    checked = {}   # head -> (abs error max, squared error sum, squared reference sum)

    def sample(seconds):
        # head evaluations of sequence 0's query rows, cycling over the heads in groups of 8
        t0 = time.perf_counter()
        done = 0
        while (time.perf_counter() - t0) < seconds:
            h0 = done % H
            hs = list(range(h0, min(H, h0 + 8)))
            ref = O.explicit_attention(W.c_host[b], W.k_host[b], qn, qr, W.wuk_host, W.wuv_host,
                                       scale=cfg.softmax_scale, base=cfg.rope_base, heads=hs, rows=rows)[key]
            if hs[0] not in checked:
                for j, h in enumerate(hs):
                    d = gpu[:, h].astype(np.float64) - ref[:, j]
                    checked[h] = (float(np.abs(d).max()), float((d * d).sum()), float((ref[:, j] ** 2).sum()))
            done += len(hs)
        el = time.perf_counter() - t0
        return (done / H) * len(rows) / el, done, el

    def tiny_full(reps=3):
        # the whole tiny fp32 workload (4 heads, 129 keys): one warm-up, then `reps` timed runs
        c0 = get_config(0)
        c, kp = G.cache_latent(c0, 0), G.cache_rope_pre(c0, 0)
        q0n, q0r = G.query_nope(c0, 0), G.query_rope_pre(c0, 0)
        wk, wv = G.weight_uk(c0), G.weight_uv(c0)
        run = lambda: O.explicit_attention(c, kp, q0n, q0r, wk, wv, scale=c0.softmax_scale,  # noqa: E731
                                           base=c0.rope_base)
        run()
        t0 = time.perf_counter()
        for _ in range(reps):
            run()
        return reps / (time.perf_counter() - t0)

    def limited(n, fn, *a):
        if threadpool_limits is None:
            return fn(*a)
        with threadpool_limits(limits=n):
            return fn(*a)

    v_all, done, el = limited(cores, sample, budget_s)
    v_one, done1, el1 = limited(1, sample, max(2.0, budget_s / 4))
    tiny_one = limited(1, tiny_full)
    tol = {"abs": 1e-5, "rel_l2": 1e-5} if cfg.dtype == "f32" else {"abs": 2e-2, "rel_l2": 1e-2}
    max_abs = max(v[0] for v in checked.values())
    rel = (sum(v[1] for v in checked.values()) / max(sum(v[2] for v in checked.values()), 1e-300)) ** 0.5
    parity = {"output": key, "sequence": b, "rows": [int(r) for r in rows], "heads_checked": len(checked),
              "max_abs_err": float(f"{max_abs:.3e}"), "rel_l2_err": float(f"{rel:.3e}"), "tolerance": tol,
              "pass": bool(max_abs <= tol["abs"] and rel <= tol["rel_l2"]),
              "against": "the GPU result of the last timed call on the same inputs"}
    return {"value": round(v_all, 4), "unit": "tokens/s", "cores": int(cores), "kind": "oracle", "parity": parity,
            "sample": f"{cfg.name}: sequence 0 ({int(W.lens[0])} keys), {len(rows)} query row(s), {done} head "
                      f"evaluations ({done / H:.1f} x all {H} heads) in {el:.1f} s of the fp64 non-absorbed oracle "
                      f"on {cores} threads; tokens/s = whole-token equivalents / s",
            "one_thread": {"value": round(v_one, 4), "unit": "tokens/s",
                           "sample": f"{done1} head evaluations in {el1:.1f} s, 1 BLAS thread",
                           "tiny_fp32_tokens_per_s": round(tiny_one, 2)}}


# ---------------------------------------------------------------------------------------------------
# other measurements

def copy_calibration(args):
    """One plain device-to-device copy kernel of known size, repeated: the counters read for it
    give the factor between FETCH_SIZE / WRITE_SIZE and the bytes really moved."""
    import torch
    _device()
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


def _clock_ghz(stamps):
    """Shader clock from per-wave (memtime, realtime) start/end pairs: cycles per 100 MHz tick."""
    import numpy as np
    s = stamps.cpu().numpy().astype(np.float64).reshape(-1, 2, 2)   # [wave][start/end][memtime, realtime]
    cyc = s[:, 1, 0] - s[:, 0, 0]
    rt = s[:, 1, 1] - s[:, 0, 1]
    ok = rt > 0
    return float(np.median(cyc[ok] / rt[ok]) * 0.1), float(np.median(cyc[ok])), float(np.median(rt[ok]) * 0.01)


def mfma_peak(args):
    """Chip-wide v_mfma_f32_32x32x16_bf16 issue at one and two waves per SIMD (one workgroup per CU),
    random bf16 operands: TFLOP/s by wall time, the shader clock it ran at (s_memtime over
    s_memrealtime), and the issue interval in cycles per MFMA per SIMD."""
    import torch

    from mla_decode_decoupled_amd import _ceilings as C

    dev = _device()
    stream = torch.cuda.current_stream(dev)
    n_wg = 256
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    res = []
    for wps, nacc in ((1, 1), (1, 4), (1, 8), (2, 4), (2, 8)):
        waves = n_wg * 4 * wps
        ops = (torch.randn((waves * 64 * 16,), generator=gen, device=dev).to(torch.bfloat16)
               .view(torch.int32).contiguous())
        stamps = torch.zeros((waves * 4,), dtype=torch.int64, device=dev)
        sink = torch.zeros((waves * 64,), dtype=torch.float32, device=dev)
        iters = max(1, 40000 // nacc)
        C.mfma(wps, nacc, n_wg, 100, ops, stamps, sink, stream.cuda_stream)   # warm-up
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        C.mfma(wps, nacc, n_wg, iters, ops, stamps, sink, stream.cuda_stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        n_mfma = waves * iters * 4 * nacc
        flops = n_mfma * 32768.0
        ghz, cyc, us = _clock_ghz(stamps)
        per_simd = iters * 4 * nacc * wps   # MFMAs issued by one SIMD
        res.append({"waves_per_simd": wps, "accumulators": nacc, "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "frac_of_2500": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                    "clock_ghz": round(ghz, 3),
                    # the kernel's wall time at the measured clock, per MFMA issued by one SIMD
                    "cycles_per_mfma_per_simd": round(ms * 1e-3 * ghz * 1e9 / per_simd, 2),
                    "ms": round(ms, 3), "median_wave_loop_us": round(us, 1)})
    # one dependent chain per wave in asm: the accumulator in VGPRs or AGPRs, alone or fed by one
    # ds_read_b128 per MFMA (the attention kernel's score chain)
    for variant, name, per_iter in ((100, "chain_vgpr_acc", 8), (101, "chain_agpr_acc", 8),
                                    (102, "chain_vgpr_acc_lds_fed", 8), (103, "chain_agpr_acc_lds_fed", 8),
                                    (104, "chain_lds_fed_waits_batched", 12), (105, "chain_one_valu_per_mfma", 8),
                                    (106, "chain_fed_by_transposed_reads", 8), (107, "two_accumulators_lds_fed", 8),
                                    (108, "four_accumulators_lds_fed", 8)):
        waves = n_wg * 4
        ops = (torch.randn((waves * 64 * 16,), generator=gen, device=dev).to(torch.bfloat16)
               .view(torch.int32).contiguous())
        stamps = torch.zeros((waves * 4,), dtype=torch.int64, device=dev)
        sink = torch.zeros((waves * 64,), dtype=torch.float32, device=dev)
        iters = 20000
        C.mfma(1, variant, n_wg, 100, ops, stamps, sink, stream.cuda_stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        C.mfma(1, variant, n_wg, iters, ops, stamps, sink, stream.cuda_stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        ghz, cyc, us = _clock_ghz(stamps)
        per_simd = iters * per_iter
        flops = waves * per_simd * 32768.0
        res.append({"variant": name, "waves_per_simd": 1, "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "clock_ghz": round(ghz, 3), "cycles_per_mfma_per_simd": round(cyc / per_simd, 2),
                    "ms": round(ms, 3)})
    # the same chains with two waves per SIMD (two 4-wave workgroups per CU)
    for variant, name in ((101, "chain_agpr_acc"), (103, "chain_agpr_acc_lds_fed"), (105, "chain_one_valu_per_mfma"),
                          (106, "chain_fed_by_transposed_reads")):
        n2 = 2 * n_wg
        waves = n2 * 4
        ops = (torch.randn((waves * 64 * 16,), generator=gen, device=dev).to(torch.bfloat16)
               .view(torch.int32).contiguous())
        stamps = torch.zeros((waves * 4,), dtype=torch.int64, device=dev)
        sink = torch.zeros((waves * 64,), dtype=torch.float32, device=dev)
        iters = 20000
        C.mfma(2, variant, n2, 100, ops, stamps, sink, stream.cuda_stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        C.mfma(2, variant, n2, iters, ops, stamps, sink, stream.cuda_stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        ghz, cyc, us = _clock_ghz(stamps)
        per_simd = iters * 8 * 2
        flops = waves * iters * 8 * 32768.0
        res.append({"variant": name, "waves_per_simd": 2, "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "clock_ghz": round(ghz, 3),
                    "cycles_per_mfma_per_simd": round(ms * 1e-3 * ghz * 1e9 / per_simd, 2), "ms": round(ms, 3)})
    print(json.dumps({"mfma_peak": res, "instruction": "v_mfma_f32_32x32x16_bf16", "workgroups": n_wg,
                      "note": "32 cycles per MFMA per SIMD is the dense peak (1024 flops/cycle/SIMD)"}), flush=True)


def lds_ceiling(args):
    """LDS read throughput: per CU and clock cycle, for the two read forms of the attention kernels,
    with one, two and four workgroups of 4 waves per CU."""
    import numpy as np
    import torch

    from mla_decode_decoupled_amd import _ceilings as C

    dev = _device()
    stream = torch.cuda.current_stream(dev)
    res = []
    iters = 20000
    for mode, name, bytes_per_read in ((0, "ds_read_b128", 16), (1, "ds_read_b64_tr_b16", 8)):
        for n_wg in (256, 512, 1024):
            stamps = torch.zeros((n_wg * 4 * 4,), dtype=torch.int64, device=dev)
            sink = torch.zeros((n_wg,), dtype=torch.int32, device=dev)
            C.lds(mode, n_wg, 10, sink, stamps, stream.cuda_stream)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            C.lds(mode, n_wg, iters, sink, stamps, stream.cuda_stream)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            ghz, cyc, _ = _clock_ghz(stamps)
            total = n_wg * 4 * iters * 8 * 64 * bytes_per_read
            cycles = ms * 1e-3 * ghz * 1e9
            res.append({"read": name, "workgroups_per_cu": n_wg // 256, "bytes_per_clk_per_cu": round(total / 256 / cycles, 1),
                        "tbs": round(total / (ms * 1e-3) / 1e12, 2), "clock_ghz": round(ghz, 3), "ms": round(ms, 3)})
    print(json.dumps({"lds_ceiling": res, "note": "bytes per clock per CU from the wall time at the measured clock"}),
          flush=True)


def stream_ceiling(args):
    """Read-only HBM streaming over 4 GiB: 16-byte vector loads (several depths and grids), and the
    attention kernel's own tile ring (36 KB tiles into LDS by global->LDS loads, 1-3 tiles in flight,
    one workgroup per CU)."""
    import torch

    from mla_decode_decoupled_amd import _ceilings as C

    dev = _device()
    stream = torch.cuda.current_stream(dev)
    total = 4 << 30
    src = torch.empty(total, dtype=torch.uint8, device=dev)
    src.view(torch.int32).random_(generator=None)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    res = []

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return sorted(out)[len(out) // 2]

    for n_wg in (256, 1024, 4096):
        per = (total // n_wg) // 16 * 16
        for depth in (4, 8, 16):
            ms = timed(lambda: C.stream(0, depth, n_wg, src, per, sink, None, stream.cuda_stream))
            res.append({"kind": "vector_loads", "workgroups": n_wg, "loads_in_flight_per_lane": depth,
                        "gbs": round(n_wg * per / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 3)})
    tile = 32 * 1152
    stamps = torch.zeros((256 * 4,), dtype=torch.int64, device=dev)
    for n_wg in (256,):
        per = (total // n_wg) // tile * tile
        for depth in (1, 2, 3):
            ms = timed(lambda: C.stream(1, depth, n_wg, src, per, sink, stamps, stream.cuda_stream))
            ghz, _, _ = _clock_ghz(stamps)
            res.append({"kind": "lds_tile_ring", "workgroups": n_wg, "tiles_in_flight": depth,
                        "gbs": round(n_wg * per / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 3),
                        "us_per_tile": round(ms * 1e3 / (per // tile), 4), "clock_ghz": round(ghz, 3)})
    best = max(r["gbs"] for r in res if r["kind"] == "vector_loads")
    print(json.dumps({"stream_ceiling": res, "bytes": total, "best_vector_gbs": best,
                      "best_vector_frac_of_8000": round(best / HBM_PEAK_GBS, 4)}), flush=True)


def prefill_crossover(args):
    """Absorbed (mla_absorb_q + mla_decode_attn + mla_out_proj) against explicit (mla_prefill_explicit)
    attention for n_q new rows per sequence, 2 sequences of 4096 keys, DeepSeek-V3 head shape."""
    import numpy as np
    import torch

    import mla_decode_decoupled_amd as mla

    dev = _device()
    stream = torch.cuda.current_stream(dev)
    bf = torch.bfloat16
    H, dc, dr, dn = 128, 512, 64, 128
    lc = mla.make_config(H, dn, dc, dr, dn, "bf16", 10000.0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    B, S = 2, 4096
    cache = torch.randn((B * S, dc + dr), generator=gen, device=dev).to(bf)
    seq_off = torch.tensor([0, S], dtype=torch.int64, device=dev)
    seq_len = torch.full((B,), S, dtype=torch.int32, device=dev)
    wuk = (torch.randn((H, dn, dc), generator=gen, device=dev) / dc ** 0.5).to(bf)
    wuv = (torch.randn((H, dn, dc), generator=gen, device=dev) / dc ** 0.5).to(bf)
    res = []
    for n_q in (16, 32, 64, 96, 128, 192, 256, 512, 1024, 2048):
        R = B * n_q
        qn = torch.randn((R, H, dn), generator=gen, device=dev).to(bf)
        qr = torch.randn((R, H, dr), generator=gen, device=dev).to(bf)
        q_pos = torch.from_numpy(np.concatenate([np.arange(S - n_q, S)] * B).astype(np.int32)).to(dev)
        qp = torch.empty((R, H, dc + dr), dtype=bf, device=dev)
        z = torch.empty((B, n_q, H, dc), dtype=torch.float32, device=dev)
        o = torch.empty((R, H, dn), dtype=bf, device=dev)
        ws = torch.empty(max(16, mla.mla_decode_attn_workspace_size(lc, B, n_q, S, 0)), dtype=torch.uint8, device=dev)
        wsx = torch.empty(max(16, mla.mla_prefill_explicit_workspace_size(lc, B, n_q, S)), dtype=torch.uint8,
                          device=dev)

        def absorbed(i):
            mla.mla_absorb_q(lc, qn, qr, q_pos, wuk, qp)
            mla.mla_decode_attn(lc, qp.view(B, n_q, H, dc + dr), cache, seq_off, seq_len, S, z, None, workspace=ws)
            mla.mla_out_proj(lc, z.view(R, H, dc), wuv, o)

        def explicit(i):
            mla.mla_prefill_explicit(lc, qn.view(B, n_q, H, dn), qr.view(B, n_q, H, dr), cache, seq_off, seq_len, S,
                                     wuk, wuv, o.view(B, n_q, H, dn), workspace=wsx)

        n = max(3, min(args.steps, 20))
        for f in (absorbed, explicit):
            f(0)
        torch.cuda.synchronize()
        ta = _stats(_events_time(stream, absorbed, n))["median"]
        tx = _stats(_events_time(stream, explicit, n))["median"]
        res.append({"n_q": n_q, "absorbed_ms": round(ta, 4), "explicit_ms": round(tx, 4),
                    "library_prefers_explicit": bool(mla.mla_prefill_prefers_explicit(lc, B, n_q, S))})
    print(json.dumps({"prefill_crossover": res, "batch": B, "keys": S, "heads": H,
                      "note": "hot inputs (one copy); median of per-call event intervals"}), flush=True)


def decode_loop(args):
    """Per-token latency of a stack of DeepSeek-V3-shaped MLA layers at batch B: every layer runs
    mla_project_inputs, mla_absorb_q, mla_decode_attn and mla_out_proj with W_O, the layer's output
    feeding the next layer; the caches are first filled by a prefill of --loop-context tokens through
    the same stack, then one captured decode step (all layers and the position advance) is replayed
    per token. The weights of 61 layers (~23 GB) are far beyond the last-level cache, so every token
    streams them from HBM."""
    import torch

    from mla_decode_decoupled_amd.decode_loop import DecodeStack, random_layers
    import mla_decode_decoupled_amd as mla
    from mla_workloads import get_config

    dev = _device()
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
        "prefill_path": stack.last_prefill_path,
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

    dev = _device()
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
    n = max(args.steps, 20)
    t_sep = _stats(_events_time(stream, lambda i: mla.mla_out_proj(lc, z, sep[i % reps][0], o, w_o=sep[i % reps][1],
                                                                    u=u), n))
    t_mer = _stats(_events_time(stream, lambda i: mla.mla_project_q(lm, zb, merged[i % reps], None, qn, None), n))
    print(json.dumps({"metric": "output side of one batch-1 decode token", "unit": "us",
                      "separate_us": round(t_sep["median"] * 1e3, 2),
                      "separate_weight_bytes": (H * dv * dc + dm * H * dv) * 2,
                      "merged_us": round(t_mer["median"] * 1e3, 2), "merged_weight_bytes": dm * H * dc * 2,
                      "calls": n, "copies": reps, "timing": "median of per-call event intervals"}), flush=True)


def a16_check(args):
    """The query side of one decode token (batch 1, DeepSeek-V3 shape, q_lora 1536), two ways:
    two-step — mla_project_q (W_UQ and W_QR from c_Q, 50.3 + 25.2 MB) then mla_absorb_q (W_UK, 16.8 MB,
               and the rotation of q_R): the library's path;
    merged   — q~ = M c_Q with the pre-multiplied M_i = W_UK,i^T W_UQ,i ([H*512 x 1536], 201 MB), run
               through the library's linear kernel (mla_project_q on a 256-head layer description of
               256-wide content heads, no position part). The merged path leaves out the position query
               (W_QR and its rotation) that the two-step path includes, which only favours it.
    Each weight set is replicated so every timed call reads its weights from HBM."""
    import torch

    import mla_decode_decoupled_amd as mla

    dev = _device()
    bf = torch.bfloat16
    H, dn, dc, dr, ql = 128, 128, 512, 64, 1536
    lc = mla.make_config(H, dn, dc, dr, dn, "bf16", 10000.0)
    lm = mla.make_config(256, 256, dc, 0, 128, "bf16", 10000.0)   # 256 x 256 = 65536 = H * d_latent outputs
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    reps = 4
    cq = torch.randn((1, ql), generator=gen, device=dev).to(bf)
    two = [((torch.randn((H * dn, ql), generator=gen, device=dev) / ql ** 0.5).to(bf),
            (torch.randn((H * dr, ql), generator=gen, device=dev) / ql ** 0.5).to(bf),
            (torch.randn((H, dn, dc), generator=gen, device=dev) / dc ** 0.5).to(bf)) for _ in range(reps)]
    merged = [(torch.randn((H * dc, ql), generator=gen, device=dev) / ql ** 0.5).to(bf) for _ in range(reps)]
    qn = torch.empty((1, H, dn), dtype=bf, device=dev)
    qr = torch.empty((1, H, dr), dtype=bf, device=dev)
    q_pos = torch.full((1,), 4096, dtype=torch.int32, device=dev)
    qp = torch.empty((1, H, dc + dr), dtype=bf, device=dev)
    qm = torch.empty((1, 256, 256), dtype=bf, device=dev)
    stream = torch.cuda.current_stream(dev)

    def two_step(i):
        wuq, wqr, wuk = two[i % reps]
        mla.mla_project_q(lc, cq, wuq, wqr, qn, qr)
        mla.mla_absorb_q(lc, qn, qr, q_pos, wuk, qp)

    n = max(args.steps, 20)
    t_two = _stats(_events_time(stream, two_step, n))
    t_mer = _stats(_events_time(stream, lambda i: mla.mla_project_q(lm, cq, merged[i % reps], None, qm, None), n))
    print(json.dumps({"metric": "query side of one batch-1 decode token (from c_Q)", "unit": "us",
                      "two_step_us": round(t_two["median"] * 1e3, 2),
                      "two_step_weight_bytes": (H * dn * ql + H * dr * ql + H * dn * dc) * 2,
                      "merged_us": round(t_mer["median"] * 1e3, 2), "merged_weight_bytes": H * dc * ql * 2,
                      "calls": n, "copies": reps, "timing": "median of per-call event intervals"}), flush=True)


if __name__ == "__main__":
    main()
