"""Plain CPU oracle of the paged cache's block manager with prefix caching.

TEST INFRASTRUCTURE ONLY. Imported by tests/; never by the library. It shares no code with
the library's native block manager; the hash comes from the ``xxhash`` package.

Source: [P1] "vLLM 学习笔记 02：nano-vllm 源码逐段精读", the Block, BlockManager and Sequence
listings and the Scheduler (schedule, preempt, postprocess) that calls them. What the
manager computes, restated:

* The pool is ``num_blocks`` blocks. Free ones wait in a FIFO (initially 0, 1, 2, ...);
  a used one counts the tables that hold it.
* Hash of block i of a token stream: XXH64 (seed 0) of the bytes of block i-1's hash
  (8 bytes, little-endian; absent for i = 0 or when block i-1 has no hash) followed by
  the block's token ids as int64 little-endian. A block keeps the hash and token ids it
  was sealed with, and an index maps each sealed hash to its block.
* ``probe`` (can_allocate): for the blocks of a sequence before its last one, in order,
  stop at the first whose hash is not indexed or whose indexed block holds other tokens;
  the blocks before that are hits. Refuse (-1) when the FIFO is shorter than the number
  of blocks the sequence needs minus its hits on used blocks; else return the hit count.
* ``admit`` (allocate) with n hits: hit blocks join the table (used ones gain a count,
  free ones leave the FIFO wherever they are and start at one); the remaining blocks are
  popped off the FIFO front, each forgetting its seal (and its index entry if the index
  still points at it). The sequence then has n * block_size cached tokens.
* ``retire`` (deallocate): table entries from last to first lose a count; a block at zero
  is pushed on the FIFO back, seal kept.
* ``room_to_grow`` / ``grow`` (can_append / may_append): a sequence whose length is 1
  modulo the block size has its newest token in a new block: one free block is needed /
  taken off the FIFO front.
* ``seal`` (hash_blocks): the blocks fully covered by cached + scheduled tokens and not by
  cached tokens alone get sealed, chaining from the block before them, and indexed
  (overwriting an index entry with the same hash).

Pins: tests/test_block_manager.py checks this against hand-derived outcomes of short
scenarios (prefix hits, shared references, revival of a freed block, eviction, the
growth rule at block boundaries) and the hash against the XXH64 test vector.

Parity unpinned: the chained hash's byte layout (the previous hash as 8 little-endian
bytes, then the token ids as int64 little-endian). The page prints no hash value, so
beyond the XXH64 specification's value for the empty input nothing outside this file fixes
the layout; it is the reading of the page's compute_hash listing (to_bytes(8, "little"),
then a numpy int64 array's bytes). The policy is pinned; only the hash bytes are not.
"""
from __future__ import annotations

from collections import deque

import numpy as np
import xxhash


def block_hash(token_ids, prefix=None) -> int:
    """XXH64 of [prefix as 8 LE bytes] + token ids as int64 LE; ``prefix`` None = no prefix."""
    h = xxhash.xxh64(seed=0)
    if prefix is not None:
        h.update(int(prefix).to_bytes(8, "little", signed=False))
    h.update(np.asarray(token_ids, dtype="<i8").tobytes())
    return h.intdigest()


class SeqState:
    def __init__(self, token_ids):
        self.tokens = [int(t) for t in token_ids]
        self.table: list[int] = []
        self.num_cached = 0
        self.num_scheduled = 0

    def nblocks(self, bs):
        return -(-len(self.tokens) // bs)

    def block_tokens(self, i, bs):
        return self.tokens[i * bs:(i + 1) * bs]


class BlockManagerOracle:
    def __init__(self, num_blocks: int, block_size: int):
        assert num_blocks >= 1 and block_size >= 2
        self.bs = block_size
        self.refs = [0] * num_blocks
        self.seal_hash: list = [None] * num_blocks      # None: not sealed
        self.seal_tokens: list = [None] * num_blocks
        self.index: dict = {}
        self.fifo = deque(range(num_blocks))
        self.in_use: set = set()

    # ------------------------------------------------------------ internal moves
    def _pop_free(self) -> int:
        bid = self.fifo.popleft()
        assert self.refs[bid] == 0
        h = self.seal_hash[bid]
        if h is not None and self.index.get(h) == bid:
            del self.index[h]
        self.seal_hash[bid] = None
        self.seal_tokens[bid] = None
        self.refs[bid] = 1
        self.in_use.add(bid)
        return bid

    def _push_free(self, bid: int):
        assert self.refs[bid] == 0
        self.in_use.discard(bid)
        self.fifo.append(bid)

    def _hits(self, s: SeqState) -> list:
        out, h = [], None
        for i in range(s.nblocks(self.bs) - 1):
            toks = s.block_tokens(i, self.bs)
            h = block_hash(toks, h)
            bid = self.index.get(h)
            if bid is None or self.seal_tokens[bid] != toks:
                break
            out.append(bid)
        return out

    # ------------------------------------------------------------ the policy
    def probe(self, s: SeqState) -> int:
        assert not s.table
        hits = self._hits(s)
        need = s.nblocks(self.bs) - sum(1 for b in hits if b in self.in_use)
        return -1 if len(self.fifo) < need else len(hits)

    def admit(self, s: SeqState, n_hits: int):
        assert not s.table
        hits = self._hits(s)[:n_hits]
        assert len(hits) == n_hits
        for bid in hits:
            if bid in self.in_use:
                self.refs[bid] += 1
            else:
                self.fifo.remove(bid)
                self.refs[bid] = 1
                self.in_use.add(bid)
            s.table.append(bid)
        while len(s.table) < s.nblocks(self.bs):
            s.table.append(self._pop_free())
        s.num_cached = n_hits * self.bs

    def retire(self, s: SeqState):
        for bid in reversed(s.table):
            self.refs[bid] -= 1
            if self.refs[bid] == 0:
                self._push_free(bid)
        s.table = []
        s.num_cached = 0
        s.num_scheduled = 0

    def room_to_grow(self, s: SeqState) -> bool:
        return len(self.fifo) >= (1 if len(s.tokens) % self.bs == 1 else 0)

    def grow(self, s: SeqState):
        if len(s.tokens) % self.bs == 1:
            s.table.append(self._pop_free())

    def seal(self, s: SeqState):
        first = s.num_cached // self.bs
        last = (s.num_cached + s.num_scheduled) // self.bs
        if first == last:
            return
        h = self.seal_hash[s.table[first - 1]] if first > 0 else None
        for i in range(first, last):
            toks = s.block_tokens(i, self.bs)
            h = block_hash(toks, h)
            bid = s.table[i]
            self.seal_hash[bid] = h
            self.seal_tokens[bid] = toks
            self.index[h] = bid

    def commit(self, s: SeqState):
        s.num_cached += s.num_scheduled
        s.num_scheduled = 0
