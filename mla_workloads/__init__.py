"""Seeded synthetic workloads for absorbed-MLA decode with decoupled RoPE.

This package only draws random inputs and rounds them to their storage dtype.
It holds none of the attention arithmetic: both the CPU oracle (``oracle/``)
and the HIP path consume what it produces, and neither imports the other.
"""

from .configs import CONFIGS, MLAConfig, get_config
from .generate import (
    TensorId,
    round_bf16,
    bf16_bits,
    seq_lens,
    cache_latent,
    cache_rope_pre,
    query_nope,
    query_rope_pre,
    weight_uk,
    weight_uv,
    weight_o,
    full_layer_inputs,
)

__all__ = [
    "CONFIGS",
    "MLAConfig",
    "get_config",
    "TensorId",
    "round_bf16",
    "bf16_bits",
    "seq_lens",
    "cache_latent",
    "cache_rope_pre",
    "query_nope",
    "query_rope_pre",
    "weight_uk",
    "weight_uv",
    "weight_o",
    "full_layer_inputs",
]
