"""float64 CPU oracle for MLA over a latent KV cache — test infrastructure only.

Only tests, the package smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the HIP library or its binding.
"""
from .mla_oracle import (  # noqa: F401
    absorbed_query, cache_rows, expand_kv, head_groups, latent, max_rel_err, mla_attention,
    mla_layer, query, rmsnorm, rope, rope_angles, rotary_key, softmax_attention, split_rows,
)
