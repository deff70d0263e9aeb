"""Seeded synthetic workloads shaped like the pages' engine runs.

A workload describes one step of the engine for one attention layer:

* ``seq_lens[b]``   tokens of sequence b once this step has run (``len(seq)``),
* ``num_cached[b]`` tokens whose K/V already sit in the paged pool before the
  step (decode: every token but the newest; prefill: the prefix-cache hit),
* ``block_tables[b]`` the physical block ids of the sequence, in logical order,
* the token values: K/V for every token of every sequence and q for the
  tokens the step computes (``seq_lens - num_cached`` per sequence).

Leading blocks may be a common prefix shared by several sequences (the prefix
cache of "vLLM 学习笔记 02：nano-vllm 源码逐段精读", BlockManager listing:
only full blocks are shared and the last block is always private). Those
tokens are stored once in ``prefix_k/prefix_v``; every other token is in the
packed ``priv_k/priv_v`` arrays, sequence by sequence, in position order.

Storage is raw: ``float32`` arrays for fp32 workloads, ``uint16`` bf16 bit
patterns for bf16 workloads. bf16 values are rounded once here, round to
nearest even, so that the oracle and the GPU consume identical inputs.

The module draws numbers and assigns block ids; it computes no slot, no
gather and no attention, so it carries none of the method's arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

BF16_POISON = np.uint16(0x7FC0)          # quiet NaN, bf16
F32_POISON = np.uint32(0x7FC00000)       # quiet NaN, fp32

CONFIG_NAMES = {
    1: "tiny_decode_b2_ctx300_700_h4kv2_d64_f32",
    2: "qwen3_0.6b_decode_b64_ctx256_4096_h16kv8_d128_bf16",
    3: "varlen_prefill_8seq_len512_2048_h16kv8_d128_bf16",
    4: "prefix_cached_prefill_32seq_prefix1024_suffix128_512_bf16",
    5: "large_decode_b512_ctx_loguniform64_4096_shared_prefix_bf16",
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


@dataclass
class Workload:
    name: str
    kind: str                      # "decode" or "prefill"
    dtype: str                     # "f32" or "bf16"
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    seq_lens: np.ndarray           # int64 [B]
    num_cached: np.ndarray         # int64 [B]
    block_tables: list             # list of int32 arrays, ceil(seq_len / block_size) ids each
    shared_blocks: np.ndarray      # int64 [B] leading blocks taken from the common prefix
    prefix_block_ids: np.ndarray   # int32 [n_prefix_blocks]
    prefix_k: np.ndarray           # raw [n_prefix_blocks * block_size, Hkv, D]
    prefix_v: np.ndarray
    priv_k: np.ndarray             # raw [sum(seq_lens - shared*bs), Hkv, D]
    priv_v: np.ndarray
    priv_off: np.ndarray           # int64 [B + 1] row offsets into priv_k / priv_v
    q: np.ndarray                  # raw [sum(seq_lens - num_cached), Hq, D]
    meta: dict = field(default_factory=dict)

    # ---- plain views over the stored arrays (no method arithmetic) ----
    @property
    def num_seqs(self) -> int:
        return int(len(self.seq_lens))

    @property
    def q_lens(self) -> np.ndarray:
        return (self.seq_lens - self.num_cached).astype(np.int64)

    @property
    def raw_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def poison_bits(self):
        return BF16_POISON if self.dtype == "bf16" else F32_POISON

    def seq_token_rows(self, b: int, lo: int, hi: int):
        """K/V rows of sequence b for positions [lo, hi) (all private positions)."""
        first = int(self.shared_blocks[b]) * self.block_size
        assert lo >= first, "positions inside the shared prefix live in prefix_k/prefix_v"
        a = int(self.priv_off[b]) + (lo - first)
        return self.priv_k[a:a + (hi - lo)], self.priv_v[a:a + (hi - lo)]

    def seq_kv_logical(self, b: int):
        """All K/V rows of sequence b in position order (prefix rows first)."""
        n_pre = int(self.shared_blocks[b]) * self.block_size
        pk, pv = self.seq_token_rows(b, n_pre, int(self.seq_lens[b]))
        return (np.concatenate([self.prefix_k[:n_pre], pk]),
                np.concatenate([self.prefix_v[:n_pre], pv]))

    def resident_segments(self):
        """(b, lo, hi) position ranges resident before the step, excluding the prefix."""
        out = []
        for b in range(self.num_seqs):
            lo = int(self.shared_blocks[b]) * self.block_size
            hi = int(self.num_cached[b])
            if hi > lo:
                out.append((b, lo, hi))
        return out

    def new_tokens(self):
        """Packed K/V of the tokens this step stores, sequence by sequence."""
        ks, vs = [], []
        for b in range(self.num_seqs):
            k, v = self.seq_token_rows(b, int(self.num_cached[b]), int(self.seq_lens[b]))
            ks.append(k)
            vs.append(v)
        shape = (0, self.num_kv_heads, self.head_dim)
        if not ks:
            return (np.zeros(shape, self.raw_dtype), np.zeros(shape, self.raw_dtype))
        return np.concatenate(ks), np.concatenate(vs)

    def max_table_len(self) -> int:
        return max((len(t) for t in self.block_tables), default=0)


def _values(rng, shape, dtype, mult=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    if dtype == "bf16":
        return bf16_round_bits(x)
    return x


def _blocks_for(n_tokens: int, bs: int) -> int:
    # number of blocks a sequence of n tokens occupies (the Sequence.num_blocks
    # property of the pages' engine); table sizing, not slot arithmetic
    return -(-int(n_tokens) // bs)


def _build(name, kind, dtype, rng, *, seq_lens, num_cached, Hq, Hkv, D, bs, num_blocks,
           scale, shared_blocks=None, n_prefix_blocks=0, q_mult=1.0, perm=None, meta=None):
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    num_cached = np.asarray(num_cached, dtype=np.int64)
    B = len(seq_lens)
    if shared_blocks is None:
        shared_blocks = np.zeros(B, dtype=np.int64)
    shared_blocks = np.asarray(shared_blocks, dtype=np.int64)
    assert np.all(num_cached <= seq_lens) and np.all(num_cached >= 0)
    assert np.all(shared_blocks * bs <= num_cached)
    assert np.all(shared_blocks <= n_prefix_blocks)
    if perm is None:
        perm = rng.permutation(num_blocks).astype(np.int32)
    need = n_prefix_blocks + sum(_blocks_for(n, bs) - int(s) for n, s in zip(seq_lens, shared_blocks))
    assert need <= num_blocks, f"pool of {num_blocks} blocks too small for {need}"
    prefix_ids = perm[:n_prefix_blocks].copy()
    cur = n_prefix_blocks
    tables = []
    for n, s in zip(seq_lens, shared_blocks):
        nb = _blocks_for(n, bs)
        own = perm[cur:cur + nb - int(s)]
        cur += nb - int(s)
        tables.append(np.concatenate([prefix_ids[:int(s)], own]).astype(np.int32))
    priv_counts = seq_lens - shared_blocks * bs
    priv_off = np.zeros(B + 1, dtype=np.int64)
    priv_off[1:] = np.cumsum(priv_counts)
    n_pre_tok = n_prefix_blocks * bs
    prefix_k = _values(rng, (n_pre_tok, Hkv, D), dtype)
    prefix_v = _values(rng, (n_pre_tok, Hkv, D), dtype)
    priv_k = _values(rng, (int(priv_off[-1]), Hkv, D), dtype)
    priv_v = _values(rng, (int(priv_off[-1]), Hkv, D), dtype)
    q = _values(rng, (int((seq_lens - num_cached).sum()), Hq, D), dtype, q_mult)
    return Workload(name=name, kind=kind, dtype=dtype, num_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, block_size=bs, num_blocks=num_blocks, scale=float(scale),
                    seq_lens=seq_lens, num_cached=num_cached, block_tables=tables,
                    shared_blocks=shared_blocks, prefix_block_ids=prefix_ids,
                    prefix_k=prefix_k, prefix_v=prefix_v, priv_k=priv_k, priv_v=priv_v,
                    priv_off=priv_off, q=q, meta=dict(meta or {}))


def make_decode(seed, ctx, *, Hq, Hkv, D, dtype="bf16", bs=256, num_blocks=None,
                scale=None, shared_blocks=None, n_prefix_blocks=0, q_mult=1.0, name="decode"):
    """One decode step: every sequence computes one new token at position ctx-1.

    ``ctx[b]`` is ``len(seq)`` and counts the new token, whose K/V the step
    stores before attending; the other ``ctx-1`` tokens are already resident.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(ctx, dtype=np.int64)
    assert np.all(ctx >= 1)
    if num_blocks is None:
        num_blocks = n_prefix_blocks + int(sum(_blocks_for(n, bs) for n in ctx)) + 1
    return _build(name, "decode", dtype, rng, seq_lens=ctx, num_cached=ctx - 1, Hq=Hq,
                  Hkv=Hkv, D=D, bs=bs, num_blocks=num_blocks,
                  scale=(1.0 / np.sqrt(D)) if scale is None else scale,
                  shared_blocks=shared_blocks, n_prefix_blocks=n_prefix_blocks, q_mult=q_mult)


def make_prefill(seed, q_lens, cached=None, *, Hq, Hkv, D, dtype="bf16", bs=256,
                 num_blocks=None, scale=None, shared_blocks=None, n_prefix_blocks=0,
                 q_mult=1.0, name="prefill"):
    """One prefill step: sequence b computes q_lens[b] tokens after cached[b] resident ones."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q_lens = np.asarray(q_lens, dtype=np.int64)
    cached = np.zeros_like(q_lens) if cached is None else np.asarray(cached, dtype=np.int64)
    seq_lens = cached + q_lens
    if num_blocks is None:
        num_blocks = n_prefix_blocks + int(sum(_blocks_for(n, bs) for n in seq_lens)) + 1
    return _build(name, "prefill", dtype, rng, seq_lens=seq_lens, num_cached=cached, Hq=Hq,
                  Hkv=Hkv, D=D, bs=bs, num_blocks=num_blocks,
                  scale=(1.0 / np.sqrt(D)) if scale is None else scale,
                  shared_blocks=shared_blocks, n_prefix_blocks=n_prefix_blocks, q_mult=q_mult)


def another_layer(w: Workload, seed: int, q_mult: float = 1.0) -> Workload:
    """The same sequences, lengths and block tables with fresh values: a second attention
    layer of the model, whose pool is indexed by the same block ids (each layer has its own
    K/V and query rows). Values from PCG64(seed), drawn as the workload's own."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return replace(
        w, name=f"{w.name}_layer{seed}",
        prefix_k=_values(rng, w.prefix_k.shape, w.dtype),
        prefix_v=_values(rng, w.prefix_v.shape, w.dtype),
        priv_k=_values(rng, w.priv_k.shape, w.dtype),
        priv_v=_values(rng, w.priv_v.shape, w.dtype),
        q=_values(rng, w.q.shape, w.dtype, q_mult), meta=dict(w.meta))


def make_config(i: int, q_mult: float = 1.0) -> Workload:
    """The five workloads the path is measured on (their stated sizes and distributions).

    Structure and values come from PCG64(1000 + i).
    """
    rng = np.random.Generator(np.random.PCG64(1000 + i))
    name = CONFIG_NAMES[i]
    if i == 1:
        perm = rng.permutation(16).astype(np.int32)
        return _build(name, "decode", "f32", rng, seq_lens=[300, 700], num_cached=[299, 699],
                      Hq=4, Hkv=2, D=64, bs=256, num_blocks=16, scale=1.0 / 8.0, perm=perm,
                      q_mult=q_mult)
    if i == 2:
        ctx = rng.integers(256, 4096, size=64, endpoint=True)
        return _build(name, "decode", "bf16", rng, seq_lens=ctx, num_cached=ctx - 1, Hq=16,
                      Hkv=8, D=128, bs=256, num_blocks=2048, scale=1.0 / np.sqrt(128.0),
                      q_mult=q_mult)
    if i == 3:
        L = rng.integers(512, 2048, size=8, endpoint=True)
        return _build(name, "prefill", "bf16", rng, seq_lens=L, num_cached=np.zeros(8, np.int64),
                      Hq=16, Hkv=8, D=128, bs=256, num_blocks=1024,
                      scale=1.0 / np.sqrt(128.0), q_mult=q_mult)
    if i == 4:
        Ls = rng.integers(128, 512, size=32, endpoint=True)
        pre = 1024
        return _build(name, "prefill", "bf16", rng, seq_lens=pre + Ls,
                      num_cached=np.full(32, pre, np.int64), Hq=16, Hkv=8, D=128, bs=256,
                      num_blocks=1024, scale=1.0 / np.sqrt(128.0),
                      shared_blocks=np.full(32, 4, np.int64), n_prefix_blocks=4, q_mult=q_mult)
    if i == 5:
        B, bs = 512, 256
        u = rng.uniform(np.log(64.0), np.log(4096.0), size=B)
        ctx = np.clip(np.rint(np.exp(u)), 64, 4096).astype(np.int64)
        sharers = rng.permutation(B)[: B // 2]
        want = rng.integers(2, 8, size=B // 2, endpoint=True)
        shared = np.zeros(B, np.int64)
        # the newest token's block is always private: at most the full blocks before it
        shared[sharers] = np.minimum(want, (ctx[sharers] - 1) // bs)
        meta = {"shared_hist": {int(k): int(v) for k, v in
                                zip(*np.unique(shared[sharers], return_counts=True))}}
        return _build(name, "decode", "bf16", rng, seq_lens=ctx, num_cached=ctx - 1, Hq=16,
                      Hkv=8, D=128, bs=bs, num_blocks=8192, scale=1.0 / np.sqrt(128.0),
                      shared_blocks=shared, n_prefix_blocks=8, q_mult=q_mult, meta=meta)
    raise ValueError(f"no config {i}")


CHUNKED_PREFILL_NAME = "chunked_prefill_16seq_cached1_2048_chunk128_1024_bf16"


def make_chunked_prefill(q_mult: float = 1.0) -> Workload:
    """Chunked prefill (the engine's prefill of a long prompt in pieces): 16 sequences whose
    first U{1..2048} tokens are already resident - cut anywhere, so the chunk's first token
    usually falls inside a block - each computing a chunk of U{128..1024} more tokens; bf16,
    16 q / 8 kv heads, head_dim 128, block 256. Structure and values from PCG64(1006)."""
    rng = np.random.Generator(np.random.PCG64(1006))
    cached = rng.integers(1, 2048, size=16, endpoint=True)
    chunk = rng.integers(128, 1024, size=16, endpoint=True)
    return _build(CHUNKED_PREFILL_NAME, "prefill", "bf16", rng, seq_lens=cached + chunk,
                  num_cached=cached, Hq=16, Hkv=8, D=128, bs=256, num_blocks=1024,
                  scale=1.0 / np.sqrt(128.0), q_mult=q_mult)
