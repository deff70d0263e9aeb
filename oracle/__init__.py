"""CPU oracle for the paged-attention path (test infrastructure only).

This package is the slow, obviously correct reference that the HIP path is
checked against. Only the tests, the smoke check and the bench's CPU-baseline
leg may import it; the library never does. It shares no code with the HIP path.
"""
from .paged_attention import (  # noqa: F401
    bf16_bits_to_f64,
    to_f64,
    prefill_metadata,
    decode_metadata,
    slot_of,
    store_kvcache,
    gather_kv,
    attend,
    softmax_probs,
    paged_attn_decode,
    paged_attn_prefill_varlen,
    attn_prefill_varlen,
)
