"""Oracle-side driver: runs one workload step entirely through ``oracle/``.

Setup (outside the step): a pool poisoned with NaN everywhere, then the
resident tokens scattered into it (the common prefix once, then each
sequence's private resident positions). The step: metadata, scatter of the new
tokens, attention. Test infrastructure only; it calls nothing from the library.
"""
from __future__ import annotations

import numpy as np

import oracle as O


def poisoned_pool(w, fill=None):
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    val = w.poison_bits() if fill is None else fill
    return np.full(shape, val, dtype=np.uint16 if w.dtype == "bf16" else np.uint32)


def as_raw(w, pool):
    """View a pool of bit patterns in the workload's raw dtype."""
    return pool if w.dtype == "bf16" else pool.view(np.float32)


def setup_pools(w, fill=None):
    kc = as_raw(w, poisoned_pool(w, fill))
    vc = as_raw(w, poisoned_pool(w, fill))
    n_pre = len(w.prefix_block_ids) * w.block_size
    if n_pre:
        md = O.prefill_metadata([n_pre], [0], [w.prefix_block_ids], w.block_size)
        O.store_kvcache(w.prefix_k, w.prefix_v, kc, vc, md["slot_mapping"])
    for b, lo, hi in w.resident_segments():
        md = O.prefill_metadata([hi], [lo], [w.block_tables[b]], w.block_size)
        k, v = w.seq_token_rows(b, lo, hi)
        O.store_kvcache(k, v, kc, vc, md["slot_mapping"])
    return kc, vc


def step_metadata(w, width=None):
    if w.kind == "decode":
        return O.decode_metadata(w.seq_lens, w.block_tables, w.block_size, width)
    return O.prefill_metadata(w.seq_lens, w.num_cached, w.block_tables, w.block_size, width)


def run_step(w, kc, vc, md=None, seqs=None):
    """Store the step's new tokens, then attend. Returns (out_f64, metadata)."""
    md = step_metadata(w) if md is None else md
    nk, nv = w.new_tokens()
    O.store_kvcache(nk, nv, kc, vc, md["slot_mapping"])
    if w.kind == "decode":
        out = O.paged_attn_decode(w.q, kc, vc, w.dtype, md["block_tables"], md["context_lens"],
                                  w.scale, w.block_size, seqs=seqs)
    else:
        out = O.paged_attn_prefill_varlen(w.q, kc, vc, w.dtype, md["block_tables"],
                                          md["cu_seqlens_q"], md["cu_seqlens_k"], w.scale,
                                          w.block_size, seqs=seqs)
    return out, md


def run_workload(w, fill=None, seqs=None):
    kc, vc = setup_pools(w, fill)
    out, md = run_step(w, kc, vc, seqs=seqs)
    return out, md, kc, vc
