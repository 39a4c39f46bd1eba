"""MLA over a compressed latent KV cache for AMD Instinct MI355X (gfx950).

The computation lives in libmla_amd.so (hand-written HIP kernels behind the C ABI
of include/mla.h); this package only loads it and marshals torch tensors into
its calls:

    mla_write_cache  — c = x·W_DKVᵀ (+RMSNorm), kr = RoPE(x·W_KRᵀ), store [c ; kr]
    mla_absorb       — q_lat = (x·W_QCᵀ)·W_UK per head, q_pe = RoPE(x·W_QRᵀ)
    mla_decode       — one query per sequence against its cached rows
    mla_decode_noalloc — mla_decode with the library's static scratch (allocates nothing)
    mla_prefill      — causal attention over packed sequences
    mla_decode_partials — the decode attention's per-split softmax partials
    mla_query        — q_nope = x·W_QCᵀ, q_pe = RoPE(x·W_QRᵀ) (no absorption)
    mla_prefill_expanded — causal prefill in the original order (k_nope, v expanded)
    mla_absorb_lowrank / mla_query_lowrank — the low-rank query path (W_QA, RMSNorm, W_QB)
    mla_output       — the output projection W_o after W_UV
    mla_tile_weights — a weight re-laid once into 24 KB blocks, read by mla_absorb_tiled,
                       mla_absorb_lowrank_tiled and mla_output_tiled (few-token steps)
    mla_rope_yarn_table — YaRN's rescaled rotary frequencies, for mla_dims.rope_freqs
    mla_v4_*         — the DeepSeek-V4 / nanowhale variant (one KV head as key and value,
                       attention sink, inverse rotation of the output, grouped output)

Build the library with ``python -m head_latent_attention_kv_amd.build``.
"""
from ._abi import (  # noqa: F401
    MLA_V4_OP_DECODE, MLA_V4_OP_OUTPUT, MLA_V4_OP_PREFILL, MLA_V4_OP_QUERY, MLA_V4_OP_WRITE_CACHE, MlaV4Dims,
    mla_v4_decode, mla_v4_output, mla_v4_prefill, mla_v4_query, mla_v4_workspace_size, mla_v4_write_cache,
    v4_dims_of,
    MLA_BF16, MLA_EHIP, MLA_EINVAL, MLA_ESCRATCH, MLA_NOALLOC_SCRATCH_BYTES, mla_decode_noalloc, MLA_ENOTSUP, MLA_EWORKSPACE, MLA_F32, MLA_OK, MLA_OP_ABSORB,
    MLA_OP_DECODE, MLA_OP_OUTPUT, MLA_OP_PREFILL, MLA_OP_PREFILL_EXPANDED, MLA_OP_QUERY, MLA_OP_WRITE_CACHE,
    MlaDims, MlaError, dims_of, load, make_dims, mla_absorb, mla_absorb_lowrank, mla_decode,
    mla_decode_partials, mla_decode_split_rows, mla_decode_splits, mla_lowrank_workspace_size, mla_output,
    mla_prefill, mla_prefill_expanded, mla_query, mla_query_lowrank, mla_rope_yarn_table, mla_workspace_size,
    mla_write_cache,
    mla_absorb_tiled, mla_absorb_lowrank_tiled, mla_output_tiled, mla_tile_weights, mla_tiled_weight_bytes,
    strerror,
)

__all__ = [
    "MlaDims", "MlaError", "dims_of", "load", "make_dims", "mla_absorb", "mla_decode",
    "mla_decode_partials", "mla_decode_noalloc", "mla_decode_split_rows", "mla_decode_splits", "mla_prefill",
    "mla_prefill_expanded", "mla_query", "mla_workspace_size", "mla_write_cache", "strerror",
    "mla_absorb_lowrank", "mla_query_lowrank", "mla_lowrank_workspace_size", "mla_output",
    "MlaV4Dims", "v4_dims_of", "mla_v4_write_cache", "mla_v4_query", "mla_v4_decode", "mla_v4_prefill",
    "mla_v4_output", "mla_v4_workspace_size",
    "mla_tile_weights", "mla_tiled_weight_bytes", "mla_absorb_tiled", "mla_output_tiled",
    "mla_absorb_lowrank_tiled",
]
