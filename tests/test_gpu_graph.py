"""Graph capture: the four C-ABI calls captured once in a HIP graph (as bench.py runs them) give,
on every replay, bit for bit what the same calls give launched eagerly. Between replays the
program refills the inputs with eager work and synchronizes, so a node that only worked on the
first replay would show up. No oracle here: the eager path is checked against the oracle by the
parity tests, and this test pins the replayed path to it."""

import pytest

torch = pytest.importorskip("torch")

import mla_decode_decoupled_amd as mla  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("batch,length", [(1, 4097), (20, 600)])
def test_graph_replay_matches_eager(batch, length):
    """batch 1 over 4097 keys takes the head-split attention kernel and the GEMV projections;
    20 rows take the MFMA attention kernel with balanced chunks and the GEMM projections."""
    dev = torch.device("cuda:0")
    H, dn, dc, dr, dv = 128, 128, 512, 64, 128
    row = dc + dr
    lc = mla.make_config(H, dn, dc, dr, dv, "bf16", 10000.0)
    bf = torch.bfloat16
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234 + batch)

    def rnd(*shape, scale=1.0):
        return (torch.randn(shape, device=dev, generator=gen) * scale).to(bf)

    B, R = batch, batch
    cache = rnd(B * length, row, scale=0.5)
    seq_off = torch.arange(B, dtype=torch.int64, device=dev) * length
    seq_len = torch.full((B,), length, dtype=torch.int32, device=dev)
    len_before = seq_len - 1
    q_pos = len_before.clone()
    c_new, k_new = rnd(B, 1, dc), rnd(B, 1, dr)
    qn, qr = rnd(R, H, dn), rnd(R, H, dr)
    wuk, wuv = rnd(H, dn, dc, scale=dc ** -0.5), rnd(H, dv, dc, scale=dc ** -0.5)
    q_packed = torch.empty((R, H, row), dtype=bf, device=dev)
    z = torch.empty((B, 1, H, dc), device=dev)
    lse = torch.empty((B, 1, H), device=dev)
    o = torch.empty((R, H, dv), dtype=bf, device=dev)
    ws = torch.empty(max(mla.mla_decode_attn_workspace_size(lc, B, 1, length, 0), 16), dtype=torch.uint8, device=dev)

    def step():
        mla.mla_rope_append(lc, c_new, k_new, cache, seq_off, len_before)
        mla.mla_absorb_q(lc, qn, qr, q_pos, wuk, q_packed)
        mla.mla_decode_attn(lc, q_packed.view(B, 1, H, row), cache, seq_off, seq_len, length, z, lse, n_splits=0,
                            workspace=ws)
        mla.mla_out_proj(lc, z.view(R, H, dc), wuv, o)

    def outputs():
        return [t.clone() for t in (q_packed, z, lse, o, cache[seq_off + len_before])]

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (c_new, k_new, qn, qr):
            t.copy_(rnd(*t.shape))
        for t in (q_packed, z, lse, o):
            t.fill_(float("nan"))
        cache[seq_off + len_before] = 0   # the replay must write the new rows itself
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = outputs()
        for t in (q_packed, z, lse, o):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        eager = outputs()
        for name, a, b in zip(("q_packed", "z", "lse", "o", "cache rows"), replayed, eager):
            assert torch.isfinite(b.float()).all(), f"replay {rep}: eager {name} not finite"
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager calls"
        print(f"replay {rep}: all outputs equal to the eager calls", flush=True)
