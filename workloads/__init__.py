"""Seeded synthetic inputs for the paged-attention path.

This package is shared by the oracle-side tests, the GPU parity tests and the
bench. It draws lengths, block-id assignments and values only: it holds none of
the attention or slot arithmetic, so neither side can inherit a mistake from it.
"""
from .synth import (  # noqa: F401
    Workload,
    CONFIG_NAMES,
    make_config,
    another_layer,
    make_decode,
    make_prefill,
    make_chunked_prefill,
    CHUNKED_PREFILL_NAME,
    bf16_round_bits,
    BF16_POISON,
    F32_POISON,
)
