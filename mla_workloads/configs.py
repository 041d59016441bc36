"""The five workload shapes: one tiny fp32 case and four DeepSeek-V3-shaped bf16 cases.

Shapes follow the DeepSeek-V2/V3 attention configuration given on the pages
("Decoupled RoPE · MLA Part 2", §6: 128 heads, 128-dim content heads, 512-dim
latent, 64-dim position part; "从零理解 MLA", section "实际配置"; query
compression to 1536 in V3 per §6 of the first page).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class MLAConfig:
    cid: int
    name: str
    batch: int
    n_heads: int
    d_model: int
    q_lora: Optional[int]
    d_latent: int
    d_rope: int
    d_nope: int
    d_v: int
    n_q: int                      # query rows per sequence (1 = decode)
    dtype: str                    # storage dtype of cache, weights, q_packed, o: "f32" | "bf16"
    rope_base: float = 10000.0
    # keys per sequence *including* the n_q new tokens; None = ragged (drawn by seq_lens())
    fixed_len: Optional[int] = None
    ragged_range: Optional[Tuple[int, int]] = None   # inclusive history-length range when ragged
    n_splits: int = 0             # split-K chunks per sequence used by the bench (0 = auto)
    latent_rms_norm: bool = True  # cache-side latent rows drawn RMS-normalised
    description: str = field(default="", compare=False)

    @property
    def row(self) -> int:
        """Elements per cached token: latent then rotated position key."""
        return self.d_latent + self.d_rope

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(d_h + d_R): the concatenated per-head query/key width
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)


CONFIGS = {
    0: MLAConfig(
        cid=0, name="tiny_fp32", batch=1, n_heads=4, d_model=64, q_lora=None,
        d_latent=32, d_rope=8, d_nope=16, d_v=16, n_q=1, dtype="f32",
        fixed_len=129, latent_rms_norm=False,
        description="Tiny fp32 decode step: 128 cached tokens at positions 0..127 plus one new query at 128",
    ),
    1: MLAConfig(
        cid=1, name="v3_decode_s4k", batch=1, n_heads=128, d_model=7168, q_lora=1536,
        d_latent=512, d_rope=64, d_nope=128, d_v=128, n_q=1, dtype="bf16",
        fixed_len=4097,
        description="DeepSeek-V3-shaped decode step, batch 1, 4096 cached tokens plus one new",
    ),
    2: MLAConfig(
        cid=2, name="v3_decode_ragged_b64", batch=64, n_heads=128, d_model=7168, q_lora=1536,
        d_latent=512, d_rope=64, d_nope=128, d_v=128, n_q=1, dtype="bf16",
        ragged_range=(1024, 8192),
        description="Batched ragged decode, 64 sequences, history lengths uniform in [1024, 8192]",
    ),
    3: MLAConfig(
        cid=3, name="v3_decode_long_b4_s128k", batch=4, n_heads=128, d_model=7168, q_lora=1536,
        d_latent=512, d_rope=64, d_nope=128, d_v=128, n_q=1, dtype="bf16",
        fixed_len=131073, n_splits=64,
        description="Long-context decode, 4 sequences of 131072 cached tokens plus one new, 64 split-K chunks",
    ),
    4: MLAConfig(
        cid=4, name="v3_chunked_prefill_b2", batch=2, n_heads=128, d_model=7168, q_lora=1536,
        d_latent=512, d_rope=64, d_nope=128, d_v=128, n_q=2048, dtype="bf16",
        fixed_len=4096,
        description="Chunked prefill, 2 sequences, 2048 new tokens after a 2048-token cached prefix",
    ),
}


def get_config(cid: int) -> MLAConfig:
    return CONFIGS[int(cid)]
