"""fp64 CPU oracle for absorbed-MLA decode with decoupled RoPE.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline leg import this package. The HIP path never does.
"""

from .mla_oracle import (  # noqa: F401
    rope_inv_freq,
    rope_rotate,
    visible,
    softmax_masked,
    explicit_attention,
    output_projection,
    absorb_query,
    cache_rows,
    packed_query,
    latent_attention,
    latent_out_projection,
    rms_norm,
    project_inputs,
    full_layer,
)
