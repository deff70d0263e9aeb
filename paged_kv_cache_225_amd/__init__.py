"""Paged-attention hot path for AMD Instinct MI355X (gfx950).

The compute lives in libpaged_kv.so (hand-written HIP kernels behind a C ABI, declared in
include/paged_kv.h). This package is the thin Python binding over it.
"""
from ._binding import (  # noqa: F401
    PKV_BF16,
    PKV_F32,
    BlockManager,
    DecodeGraphs,
    PagedKVError,
    PreconditionError,
    attn_prefill_varlen,
    load_library,
    paged_attn_decode,
    paged_attn_decode_noalloc,
    paged_attn_decode_prefix,
    paged_attn_decode_prefix_workspace_bytes,
    prefix_groups,
    paged_attn_decode_store,
    paged_attn_decode_workspace_bytes,
    paged_attn_prefill_varlen,
    pkv_block_hash,
    pkv_check_decode,
    pkv_check_prefix,
    pkv_check_prefill,
    pkv_check_store,
    pkv_decode_metadata,
    pkv_prefill_metadata,
    pkv_sample,
    pkv_sample_workspace_bytes,
    pkv_status_string,
    pkv_xxh64,
    store_kvcache,
)

__all__ = [
    "PKV_BF16", "PKV_F32", "BlockManager", "DecodeGraphs", "PagedKVError", "attn_prefill_varlen",
    "load_library", "paged_attn_decode", "paged_attn_decode_noalloc", "paged_attn_decode_prefix",
    "paged_attn_decode_prefix_workspace_bytes", "prefix_groups", "paged_attn_decode_store",
    "paged_attn_decode_workspace_bytes", "paged_attn_prefill_varlen", "pkv_decode_metadata",
    "pkv_block_hash", "pkv_prefill_metadata", "pkv_sample", "pkv_sample_workspace_bytes",
    "pkv_status_string", "pkv_xxh64", "store_kvcache", "PreconditionError", "pkv_check_decode",
    "pkv_check_prefill", "pkv_check_prefix", "pkv_check_store",
]
