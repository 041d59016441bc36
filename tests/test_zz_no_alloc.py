"""mla_decode_step_noalloc through the C ABI against mla_decode_step on the same inputs: two calls
in a row on the batch-1 DeepSeek-V3-shaped decode step (4097 keys), then a smaller step (1500 keys,
another split plan over the same scratch), then the tiny fp32 workload (the generic kernels'
partials in the scratch). Every output must equal mla_decode_step's bit for bit (same kernels, same
plan), and the first step's must meet the oracle bar."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from mla_workloads import MLAConfig, get_config  # noqa: E402

from .gpu_pipeline import assert_close, host_inputs, np32, run_step  # noqa: E402

import oracle as O  # noqa: E402


def _same(a, b, what):
    for name in ("cache", "q_packed", "z", "lse", "o"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.uint8) if y.dtype != torch.float32 else y.view(torch.int32)), \
            f"{what}: {name} differs from mla_decode_step's"


def test_noalloc_step_matches_step_twice_then_smaller():
    cfg = get_config(1)
    hi = host_inputs(cfg)
    print("call 1 and 2: v3_decode_s4k (4097 keys)", flush=True)
    want = run_step(hi)
    for call in (1, 2):
        got = run_step(hi, noalloc=True)
        _same(got, want, f"call {call}")
    ref = O.explicit_attention(hi.c[0], hi.k_pre[0], hi.q_nope[0], hi.q_rope[0], hi.w_uk, hi.w_uv,
                               scale=cfg.softmax_scale, base=cfg.rope_base)
    assert_close(np32(got.o[0]), ref["o"], "bf16", "noalloc o vs oracle")
    assert_close(np32(got.z[0]), ref["z"], "bf16", "noalloc z vs oracle")

    print("call 3: 1500 keys", flush=True)
    small = host_inputs(cfg, lens=[1500])
    _same(run_step(small, noalloc=True), run_step(small), "smaller step")

    print("call 4: tiny fp32, 7 splits", flush=True)
    tiny = host_inputs(get_config(0))
    _same(run_step(tiny, n_splits=7, noalloc=True), run_step(tiny, n_splits=7), "tiny fp32 step")
