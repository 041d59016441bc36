"""MI355X-native absorbed MLA decode with decoupled RoPE.

The compute path is libmla.so (HIP kernels for gfx950, C ABI in include/mla.h);
``ops`` holds thin torch wrappers with the same names as the C entry points.
"""

from .ops import (  # noqa: F401
    make_config,
    storage_dtype,
    mla_rope_append,
    mla_absorb_q,
    mla_decode_attn_workspace_size,
    mla_decode_attn,
    mla_out_proj,
    mla_decode_step_workspace_size,
    mla_decode_step,
    mla_decode_step_noalloc,
    mla_project_workspace_size,
    mla_project_kv_append,
    mla_project_q,
    mla_project_inputs_workspace_size,
    mla_project_inputs,
    mla_decode_advance,
    mla_prefill_explicit_workspace_size,
    mla_prefill_explicit,
    mla_prefill_prefers_explicit,
    version,
)
