"""Host-side checks of the seeded input generators."""

import numpy as np
import pytest

from mla_workloads import CONFIGS, get_config
from mla_workloads import generate as G


def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0], dtype=np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(G.round_bf16(x), ref)


def test_bf16_bits_roundtrip_and_rejects_unrounded():
    x = G.round_bf16(np.linspace(-3, 3, 101, dtype=np.float32))
    bits = G.bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, x)
    with pytest.raises(ValueError):
        G.bf16_bits(np.array([1.0 + 2 ** -20], dtype=np.float32))


def test_generators_are_deterministic_and_independent():
    cfg = get_config(0)
    a = G.cache_latent(cfg, 0)
    b = G.cache_latent(cfg, 0)
    assert np.array_equal(a, b)
    assert not np.array_equal(G.query_nope(cfg, 0).ravel()[:16], G.query_rope_pre(cfg, 0).ravel()[:16])


def test_shapes_and_storage_dtype():
    cfg = get_config(1)
    c = G.cache_latent(cfg, 0, n=64)
    assert c.shape == (64, 512) and c.dtype == np.float32
    assert np.all(G.bf16_bits(c) == G.bf16_bits(c))  # representable
    rms = np.sqrt(np.mean(c.astype(np.float64) ** 2, axis=1))
    assert np.allclose(rms, 1.0, atol=1e-2)
    assert G.weight_uk(cfg).shape == (128, 128, 512)
    assert G.weight_uv(cfg).shape == (128, 128, 512)
    assert G.query_nope(cfg, 0).shape == (1, 128, 128)
    assert G.query_rope_pre(cfg, 0).shape == (1, 128, 64)


def test_sequence_lengths():
    assert list(G.seq_lens(CONFIGS[0])) == [129]
    assert list(G.seq_lens(CONFIGS[1])) == [4097]
    assert list(G.seq_lens(CONFIGS[3])) == [131073] * 4
    assert list(G.seq_lens(CONFIGS[4])) == [4096, 4096]
    lens = G.seq_lens(CONFIGS[2])
    assert lens.shape == (64,) and lens.min() >= 1025 and lens.max() <= 8193
    assert np.array_equal(lens, G.seq_lens(CONFIGS[2]))
