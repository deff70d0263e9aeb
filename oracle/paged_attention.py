"""Plain fp64 CPU oracle for the paged-attention path.

TEST INFRASTRUCTURE ONLY. Imported by tests/, by the smoke check and by the
bench's CPU-baseline leg; never by the library. It shares no code, header,
table or helper with the HIP path.

Sources (the pages this follows):
  [P1] "vLLM 学习笔记 02：nano-vllm 源码逐段精读": listings ``ModelRunner.prepare_prefill``,
       ``prepare_block_tables``, ``prepare_decode``, ``store_kvcache`` / ``store_kvcache_kernel``,
       ``Attention.forward``, ``Sequence.num_blocks`` / ``last_block_num_tokens``.
  [P2] "Nano-vLLM代码手撕笔记": section "请求执行 – 输入序列预处理与context构建" (worked
       example), section "请求执行 – run model" (attention dispatch).
  [P3] "Nano-vLLM 代码解析": section 4.2.1 输入准备.

Every function is the plain definition of what the path computes:
  * metadata: one slot per position, slot = block_table[pos // bs] * bs + pos % bs;
  * scatter: a bitwise row copy per token, slot -1 skipped;
  * attention: per sequence, rebuild contiguous K/V from the block table, then
    textbook softmax(scale * q K^T) V in float64 with the causal rule that
    query i of a sequence with Lq queries and Lk keys sits at position
    Lk - Lq + i and sees keys 0..Lk-Lq+i (bottom-right alignment).

Readings where the pages are silent (each is listed with its support in the
design notes): GQA maps q head h to kv head h // (Hq / Hkv); a decode row with
context length 0 yields zeros; duplicate non-negative slots in one store are
rejected; the paged prefill always reads K/V through the block table, and the packed
form (no block table) takes sequence b's keys from rows cu_k[b]..cu_k[b+1]-1.

Pins: tests/test_oracle_pins.py checks every function here against the pages'
worked example, pure-Python brute force, closed forms, torch's fp64 SDPA and
invariants. Nothing here is parity-unpinned.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# value decoding
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# a0: host metadata  ([P1] prepare_prefill / prepare_block_tables / prepare_decode)
# --------------------------------------------------------------------------
def slot_of(block_table, pos: int, block_size: int) -> int:
    """Physical slot of logical position ``pos``: block ``block_table[pos // bs]``, offset ``pos % bs``.

    [P1] prepare_prefill builds the slot range of each block as
    ``block_table[i] * block_size`` plus the in-block offset; [P2] section
    "请求执行 – 输入序列预处理与context构建" explains slot ids as global, one per token.
    """
    return int(block_table[pos // block_size]) * block_size + pos % block_size


def _pad_tables(block_tables, width=None) -> np.ndarray:
    """[P1] prepare_block_tables: rows padded with -1 to the longest table (or ``width``)."""
    longest = max((len(t) for t in block_tables), default=0)
    width = longest if width is None else width
    if width < longest:
        raise ValueError("block-table width shorter than a table")
    out = np.full((len(block_tables), width), -1, dtype=np.int32)
    for b, t in enumerate(block_tables):
        out[b, :len(t)] = np.asarray(t, dtype=np.int32)
    return out


def _num_blocks(n_tokens: int, block_size: int) -> int:
    """[P1] Sequence.num_blocks: blocks needed for n tokens (ceiling division)."""
    return (n_tokens + block_size - 1) // block_size


def prefill_metadata(seq_lens, num_cached, block_tables, block_size, width=None) -> dict:
    """Attention metadata of a prefill step ([P1] prepare_prefill; [P2] worked example).

    Sequence b computes positions ``start = num_cached[b]`` .. ``end - 1`` with
    ``end = seq_lens[b]``: ``seqlen_q = end - start``, ``seqlen_k = end``. The slot
    mapping covers only those positions, so ``start`` may fall inside a block.
    """
    cu_q, cu_k = [0], [0]
    max_q = max_k = 0
    slots, positions = [], []
    for n, start, table in zip(seq_lens, num_cached, block_tables):
        n, start = int(n), int(start)
        if len(table) < _num_blocks(n, block_size):
            raise ValueError("block table too short for the sequence")
        seqlen_q, seqlen_k = n - start, n
        cu_q.append(cu_q[-1] + seqlen_q)
        cu_k.append(cu_k[-1] + seqlen_k)
        max_q, max_k = max(max_q, seqlen_q), max(max_k, seqlen_k)
        for pos in range(start, n):
            positions.append(pos)
            slots.append(slot_of(table, pos, block_size))
    return {
        "cu_seqlens_q": np.asarray(cu_q, dtype=np.int32),
        "cu_seqlens_k": np.asarray(cu_k, dtype=np.int32),
        "max_seqlen_q": max_q,
        "max_seqlen_k": max_k,
        "slot_mapping": np.asarray(slots, dtype=np.int32),
        "positions": np.asarray(positions, dtype=np.int64),
        "block_tables": _pad_tables(block_tables, width),
    }


def decode_metadata(seq_lens, block_tables, block_size, width=None) -> dict:
    """Attention metadata of a decode step ([P1] prepare_decode; [P2] worked example).

    Each sequence computes its newest token, position ``len(seq) - 1``, whose
    K/V goes to the last slot the sequence occupies; ``context_lens = len(seq)``
    counts that token. The table must hold exactly ``ceil(len / bs)`` blocks, so
    its last entry is the block of the newest token.
    """
    slots, ctx, positions = [], [], []
    for n, table in zip(seq_lens, block_tables):
        n = int(n)
        if n < 1 or len(table) != _num_blocks(n, block_size):
            raise ValueError("decode needs len >= 1 and exactly ceil(len/bs) blocks")
        positions.append(n - 1)
        ctx.append(n)
        slots.append(slot_of(table, n - 1, block_size))
    return {
        "slot_mapping": np.asarray(slots, dtype=np.int32),
        "context_lens": np.asarray(ctx, dtype=np.int32),
        "positions": np.asarray(positions, dtype=np.int64),
        "block_tables": _pad_tables(block_tables, width),
    }


# --------------------------------------------------------------------------
# a1: scatter  ([P1] store_kvcache / store_kvcache_kernel)
# --------------------------------------------------------------------------
def store_kvcache(key, value, k_cache, v_cache, slot_mapping) -> None:
    """Copy token t's K and V rows (all kv heads, bit for bit) into slot ``slot_mapping[t]``.

    ``key``/``value`` are [N, Hkv, D] raw arrays (any token stride); the caches are
    raw [num_blocks, block_size, Hkv, D] arrays, updated in place. Slot -1 means
    "do not store" ([P1] kernel returns early; [P2] notes padding / prefix reuse).
    Untouched slots keep their bytes. Non-negative slots must be unique and in range.
    """
    slot_mapping = np.asarray(slot_mapping)
    N = key.shape[0]
    if slot_mapping.shape != (N,) or value.shape[0] != N:
        raise ValueError("slot_mapping must have one entry per token")
    kflat = k_cache.reshape(-1, k_cache.shape[2] * k_cache.shape[3])
    vflat = v_cache.reshape(-1, v_cache.shape[2] * v_cache.shape[3])
    used = [int(s) for s in slot_mapping if s != -1]
    if len(set(used)) != len(used):
        raise ValueError("duplicate slots in one store")
    for t in range(N):
        s = int(slot_mapping[t])
        if s == -1:
            continue
        if not 0 <= s < kflat.shape[0]:
            raise ValueError("slot out of range")
        kflat[s, :] = key[t].reshape(-1)
        vflat[s, :] = value[t].reshape(-1)


# --------------------------------------------------------------------------
# gather + attention  ([P1] Attention.forward; [P2] "请求执行 – run model")
# --------------------------------------------------------------------------
def gather_kv(cache, dtype: str, block_table, n_keys: int, block_size: int) -> np.ndarray:
    """Contiguous [n_keys, Hkv, D] float64 rows of one sequence: key j sits in
    block ``block_table[j // bs]`` at offset ``j % bs``. Entries past the
    sequence's blocks are never read."""
    j = np.arange(n_keys)
    blocks = np.asarray(block_table, dtype=np.int64)[j // block_size]
    return to_f64(cache[blocks, j % block_size], dtype)


def softmax_probs(q_rows, K, V, q_positions, scale):
    """Attention weights P[h, i, j] (textbook softmax over the visible keys)."""
    nq, Hq, _ = q_rows.shape
    nk, Hkv, _ = K.shape
    G = Hq // Hkv
    P = np.zeros((Hq, nq, nk))
    visible = np.arange(nk)[None, :] <= np.asarray(q_positions)[:, None]
    for h in range(Hq):
        g = h // G
        S = scale * (q_rows[:, h, :] @ K[:, g, :].T)
        S = np.where(visible, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        w = np.exp(S - m)
        P[h] = w / w.sum(axis=1, keepdims=True)
    return P


def attend(q_rows, K, V, q_positions, scale) -> np.ndarray:
    """out[i, h] = sum_j softmax_j(scale * <q[i,h], K[j, h//G]>) V[j, h//G] over keys j <= pos_i."""
    nq, Hq, D = q_rows.shape
    nk, Hkv, _ = K.shape
    if Hq % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    out = np.zeros((nq, Hq, D))
    if nq == 0 or nk == 0:
        return out
    P = softmax_probs(q_rows, K, V, q_positions, scale)
    G = Hq // Hkv
    for h in range(Hq):
        out[:, h, :] = P[h] @ V[:, h // G, :]
    return out


def paged_attn_decode(q, k_cache, v_cache, dtype, block_tables, context_lens, scale,
                      block_size, seqs=None) -> np.ndarray:
    """Decode attention ([P1] Attention.forward, decode branch).

    Sequence b's single query sits at position ``context_lens[b] - 1`` and attends
    all ``context_lens[b]`` keys, the newest included (its K/V is stored first).
    A row with context length 0 yields zeros. ``seqs`` restricts the work to a
    subset of rows (the others stay zero), for sampled checks at full size.
    """
    q = to_f64(q, dtype)
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in (range(B) if seqs is None else seqs):
        n = int(context_lens[b])
        if n == 0:
            continue
        K = gather_kv(k_cache, dtype, block_tables[b], n, block_size)
        V = gather_kv(v_cache, dtype, block_tables[b], n, block_size)
        out[b] = attend(q[b:b + 1], K, V, [n - 1], scale)[0]
    return out


def attn_prefill_varlen(q, k, v, dtype, cu_seqlens_q, cu_seqlens_k, scale, seqs=None) -> np.ndarray:
    """Causal varlen prefill over packed K/V rows, no block table ([P1] Attention.forward,
    prefill branch when the context carries no block tables: the step's own k and v).

    Sequence b owns query rows ``cu_q[b]..cu_q[b+1]-1`` and key/value rows
    ``cu_k[b]..cu_k[b+1]-1`` of ``k`` / ``v`` ([total_k, Hkv, D]); with ``Lq`` queries and
    ``Lk`` keys, query i sits at position ``Lk - Lq + i`` as in the paged form.
    """
    q = to_f64(q, dtype)
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D))
    B = len(cu_seqlens_q) - 1
    for b in (range(B) if seqs is None else seqs):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0:
            continue
        if Lk < Lq:
            raise ValueError("a sequence has fewer keys than queries")
        K = to_f64(k[k0:k1], dtype)
        V = to_f64(v[k0:k1], dtype)
        out[q0:q1] = attend(q[q0:q1], K, V, Lk - Lq + np.arange(Lq), scale)
    return out


def paged_attn_prefill_varlen(q, k_cache, v_cache, dtype, block_tables, cu_seqlens_q,
                              cu_seqlens_k, scale, block_size, seqs=None) -> np.ndarray:
    """Causal varlen prefill over the paged cache ([P1] Attention.forward, prefill branch).

    Sequence b owns query rows ``cu_q[b]..cu_q[b+1]-1`` and ``Lk = cu_k[b+1]-cu_k[b]``
    keys read through its block table; with ``Lq`` queries, query i sits at
    position ``Lk - Lq + i`` ([P1] prepare_prefill: positions run from the cached
    count to the end; [P2] comment Q=[CDEF], K=[ABCDEF]).
    """
    q = to_f64(q, dtype)
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D))
    B = len(cu_seqlens_q) - 1
    for b in (range(B) if seqs is None else seqs):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        Lq, Lk = q1 - q0, int(cu_seqlens_k[b + 1]) - int(cu_seqlens_k[b])
        if Lq == 0:
            continue
        if Lk < Lq:
            raise ValueError("a sequence has fewer keys than queries")
        K = gather_kv(k_cache, dtype, block_tables[b], Lk, block_size)
        V = gather_kv(v_cache, dtype, block_tables[b], Lk, block_size)
        out[q0:q1] = attend(q[q0:q1], K, V, Lk - Lq + np.arange(Lq), scale)
    return out
