"""The host block manager: the oracle pinned to hand-derived outcomes of the policy in
[P1] "vLLM 学习笔记 02：nano-vllm 源码逐段精读" (BlockManager, Scheduler), then the native
manager (pkv_bm_*) checked against the oracle, bit for bit, under a scheduler-driven
random workload (prefix sharing, chunked prefill, decode growth, preemption, finishing).
"""
from __future__ import annotations

import collections

import numpy as np
import pytest
import xxhash

from oracle.block_manager import BlockManagerOracle, SeqState, block_hash
from paged_kv_cache_225_amd import _binding as B


# ------------------------------------------------------------------ hash pins
def test_xxh64_published_vector_and_library():
    # the XXH64 specification's value for empty input with seed 0
    assert B.pkv_xxh64(b"") == 0xEF46DB3751D8E999
    assert xxhash.xxh64(b"").intdigest() == 0xEF46DB3751D8E999
    rng = np.random.Generator(np.random.PCG64(3))
    for n in list(range(0, 70)) + [255, 256, 1000, 4096]:
        d = rng.integers(0, 256, size=n, dtype=np.uint8).tobytes()
        for seed in (0, 1, 2**64 - 1):
            assert B.pkv_xxh64(d, seed) == xxhash.xxh64(d, seed=seed).intdigest()


def test_block_hash_chain():
    rng = np.random.Generator(np.random.PCG64(4))
    toks = rng.integers(0, 2**31, size=(5, 16))
    h = None
    for row in toks:
        got = B.pkv_block_hash(row, h)
        assert got == block_hash(row, h)
        h = got
    # the chain: a block's hash depends on every earlier block
    a = block_hash(toks[1], block_hash(toks[0]))
    b = block_hash(toks[1], block_hash(toks[0] + 1))
    assert a != b and block_hash(toks[1]) not in (a, b)
    # negative and large token ids are 64-bit two's complement
    assert B.pkv_block_hash([-1, 2**40]) == block_hash([-1, 2**40])


# ------------------------------------------------------------------ oracle pins
def _prefill_all(m, s):
    s.num_scheduled = len(s.tokens) - s.num_cached
    m.seal(s)
    m.commit(s)


def test_oracle_prefix_hit_shares_and_revives_blocks():
    m = BlockManagerOracle(10, 4)
    a = SeqState(range(1, 11))                  # 10 tokens: blocks [1..4] [5..8] [9 10]
    assert m.probe(a) == 0
    m.admit(a, 0)
    assert a.table == [0, 1, 2] and list(m.fifo) == [3, 4, 5, 6, 7, 8, 9]
    _prefill_all(m, a)                          # blocks 0 and 1 complete: sealed
    assert m.seal_hash[0] == block_hash([1, 2, 3, 4])
    assert m.seal_hash[1] == block_hash([5, 6, 7, 8], m.seal_hash[0])
    assert m.seal_hash[2] is None

    b = SeqState(list(range(1, 9)) + [99, 100, 101])
    assert m.probe(b) == 2                      # two hits, both in use: one new block
    m.admit(b, 2)
    assert b.table == [0, 1, 3] and b.num_cached == 8
    assert m.refs[:4] == [2, 2, 1, 1]

    m.retire(a)                                 # last entry first: 2 freed, 1 and 0 shared
    assert list(m.fifo) == [4, 5, 6, 7, 8, 9, 2] and m.refs[:4] == [1, 1, 0, 1]
    m.retire(b)
    assert list(m.fifo) == [4, 5, 6, 7, 8, 9, 2, 3, 1, 0]

    c = SeqState(list(range(1, 9)) + [50])      # hits on two free blocks: they are revived
    assert m.probe(c) == 2
    m.admit(c, 2)
    assert c.table == [0, 1, 4] and list(m.fifo) == [5, 6, 7, 8, 9, 2, 3]
    assert m.refs[0] == m.refs[1] == m.refs[4] == 1


def test_oracle_last_block_is_never_a_hit_and_needs_free_blocks():
    m = BlockManagerOracle(4, 4)
    a = SeqState(range(8))                      # exactly two full blocks
    m.admit(a, m.probe(a))
    _prefill_all(m, a)
    assert a.table == [0, 1] and m.seal_hash[1] is not None
    b = SeqState(range(8))                      # same tokens: only block 0 may be a hit
    assert m.probe(b) == 1
    c = SeqState(range(100, 113))               # 4 blocks, 2 free: refused
    assert m.probe(c) == -1
    d = SeqState(list(range(4)) + list(range(200, 209)))  # 1 hit on a used block: 3 new > 2
    assert m.probe(d) == -1
    e = SeqState(list(range(4)) + list(range(200, 205)))  # 1 hit + 2 new = fits
    assert m.probe(e) == 1


def test_oracle_handing_out_a_freed_block_evicts_its_hash():
    m = BlockManagerOracle(3, 2)
    a = SeqState([7, 7, 8])
    m.admit(a, m.probe(a))
    _prefill_all(m, a)
    h0 = m.seal_hash[0]
    m.retire(a)
    assert m.index[h0] == 0 and list(m.fifo) == [2, 1, 0]
    x = SeqState([1, 2, 3, 4, 5])               # takes 2, 1, 0: block 0 forgets [7, 7]
    m.admit(x, m.probe(x))
    assert x.table == [2, 1, 0] and h0 not in m.index and m.seal_hash[0] is None
    m.retire(x)
    y = SeqState([7, 7, 9])
    assert m.probe(y) == 0


def test_oracle_token_check_guards_the_hash_index():
    m = BlockManagerOracle(6, 2)
    a = SeqState([1, 2, 3])
    m.admit(a, m.probe(a))
    _prefill_all(m, a)
    h = m.seal_hash[0]
    m.seal_tokens[0] = [1, 5]                   # an index entry whose tokens differ
    b = SeqState([1, 2, 3])
    assert m.probe(b) == 0
    m.seal_tokens[0] = [1, 2]
    assert m.probe(b) == 1 and m.index[h] == 0


def test_oracle_growth_rule_at_block_boundaries():
    m = BlockManagerOracle(4, 4)
    s = SeqState(range(4))
    m.admit(s, m.probe(s))
    _prefill_all(m, s)
    grows = []
    for t in range(4, 16):                      # lengths 5..16
        s.tokens.append(t)
        grows.append(len(s.table) + 1 if len(s.tokens) % 4 == 1 else len(s.table))
        assert m.room_to_grow(s)
        m.grow(s)
        assert len(s.table) == grows[-1]
        s.num_scheduled = 1
        m.seal(s)
        m.commit(s)
    # lengths 5, 9 and 13 open a block; the pool of four is then used up
    assert grows == [2, 2, 2, 2, 3, 3, 3, 3, 4, 4, 4, 4] and not m.fifo
    assert all(m.seal_hash[b] is not None for b in s.table)  # 16 tokens: all four sealed
    assert m.room_to_grow(s)                    # length 16: no new block needed
    s.tokens.append(16)                         # length 17 would need a fifth block
    assert not m.room_to_grow(s)


def test_oracle_seal_chains_from_the_previous_block_across_steps():
    m = BlockManagerOracle(8, 4)
    s = SeqState(range(14))
    m.admit(s, m.probe(s))
    for n in (5, 6, 3):                          # chunked prefill: 5 + 6 + 3 tokens
        s.num_scheduled = n
        m.seal(s)
        m.commit(s)
    h = None
    for i in range(3):                           # 14 tokens: three full blocks sealed
        h = block_hash(list(range(4 * i, 4 * i + 4)), h)
        assert m.seal_hash[s.table[i]] == h
    assert m.seal_hash[s.table[3]] is None


# ------------------------------------------------------------------ native vs oracle
def _state(m_nat, m_or, seqs):
    assert m_nat.free_block_ids() == list(m_or.fifo)
    for bid in range(len(m_or.refs)):
        rc, sealed, h = m_nat.block_info(bid)
        assert rc == m_or.refs[bid], bid
        assert h == m_or.seal_hash[bid], bid
    for sid, s in seqs.items():
        assert m_nat.block_table(sid) == s.table
        info = m_nat.sequence_info(sid)
        assert info["num_cached_tokens"] == s.num_cached
        assert info["num_tokens"] == len(s.tokens)


def _drive(seed, num_blocks, bs):
    """A scheduler in the pages' shape drives both managers with the same decisions: admit
    waiting sequences (prefix hits, chunked prefill under a token budget), decode running
    ones (grow or preempt the newest), seal and commit after each step, finish sequences
    at their target length. Every observable must agree after every step."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nat = B.BlockManager(num_blocks, bs)
    orc = BlockManagerOracle(num_blocks, bs)
    prompts = [list(rng.integers(0, 50, size=int(rng.integers(1, 3 * bs)))) for _ in range(4)]
    waiting, running = collections.deque(), collections.deque()
    seqs, target = {}, {}
    budget, max_seqs = 2 * bs, 4
    seen = collections.Counter()
    for step in range(120):
        if rng.random() < 0.3 and len(seqs) < 40:   # a new request: shared prompt + own tail
            base = prompts[int(rng.integers(0, len(prompts)))]
            toks = base[: int(rng.integers(0, len(base) + 1))] + list(
                rng.integers(0, 50, size=int(rng.integers(1, 2 * bs))))
            sid = nat.add_sequence(toks)
            seqs[sid] = SeqState(toks)
            target[sid] = len(toks) + int(rng.integers(1, 3 * bs))
            waiting.append(sid)
        scheduled = []
        used = 0
        while waiting and len(scheduled) < max_seqs:       # prefill first
            sid = waiting[0]
            s = seqs[sid]
            if not s.table:
                hits = orc.probe(s)
                assert nat.can_allocate(sid) == hits
                if hits == -1:
                    seen["refused"] += 1
                    break
                seen["hits"] += hits
                n_tok = len(s.tokens) - hits * bs
            else:
                n_tok = len(s.tokens) - s.num_cached
            room = budget - used
            if room <= 0 or (room < n_tok and scheduled):
                break
            if not s.table:
                orc.admit(s, hits)
                nat.allocate(sid, hits)
            s.num_scheduled = min(n_tok, room)
            seen["chunked"] += s.num_scheduled < n_tok
            nat.set_scheduled(sid, s.num_scheduled)
            used += s.num_scheduled
            if s.num_cached + s.num_scheduled == len(s.tokens):
                waiting.popleft()
                running.append(sid)
            scheduled.append(sid)
        prefill = bool(scheduled)
        if not prefill:                                     # then decode
            while running and len(scheduled) < max_seqs:
                sid = running.popleft()
                s = seqs[sid]
                ok = orc.room_to_grow(s)
                assert nat.can_append(sid) == ok
                while not ok:
                    victim = running.pop() if running else sid
                    seen["preempted"] += 1
                    orc.retire(seqs[victim])
                    nat.deallocate(victim)
                    waiting.appendleft(victim)
                    if victim == sid:
                        break
                    ok = orc.room_to_grow(s)
                    assert nat.can_append(sid) == ok
                if not ok:
                    break
                s.num_scheduled = 1
                nat.set_scheduled(sid, 1)
                orc.grow(s)
                nat.may_append(sid)
                scheduled.append(sid)
            running.extendleft(reversed(scheduled))
        for sid in scheduled:                               # postprocess
            s = seqs[sid]
            orc.seal(s)
            nat.hash_blocks(sid)
            orc.commit(s)
            nat.commit_scheduled(sid)
            if prefill and s.num_cached < len(s.tokens):
                continue
            tok = int(rng.integers(0, 50))
            s.tokens.append(tok)
            nat.append_token(sid, tok)
            if len(s.tokens) >= target[sid]:
                orc.retire(s)
                nat.deallocate(sid)
                running.remove(sid)
                nat.remove_sequence(sid)
                del seqs[sid]
        _state(nat, orc, seqs)
    nat.close()
    print(dict(seen))
    return seen


@pytest.mark.parametrize("seed,num_blocks,bs", [(0, 24, 4), (1, 40, 8), (2, 12, 2), (3, 64, 16),
                                                (4, 16, 4)])
def test_native_matches_oracle_under_a_scheduler(seed, num_blocks, bs):
    seen = _drive(seed, num_blocks, bs)
    # the workload reaches the interesting paths
    assert seen["hits"] > 0 and seen["chunked"] > 0


def test_scheduler_workload_reaches_preemption():
    total = collections.Counter()
    for seed, nb, bs in [(0, 24, 4), (2, 12, 2), (4, 16, 4), (5, 10, 4)]:
        total += _drive(seed, nb, bs)
    assert total["preempted"] > 0 and total["refused"] > 0


def test_native_argument_errors():
    with pytest.raises(B.PagedKVError):
        B.BlockManager(0, 4)
    with pytest.raises(B.PagedKVError):
        B.BlockManager(4, 1)
    m = B.BlockManager(2, 4)
    sid = m.add_sequence([1, 2, 3, 4, 5, 6, 7, 8, 9])    # needs 3 blocks of 2
    assert m.can_allocate(sid) == -1
    with pytest.raises(B.PagedKVError):
        m.allocate(sid, 0)                                # free list too short
    with pytest.raises(B.PagedKVError):
        m.allocate(sid, 1)                                # not a hit
    with pytest.raises(B.PagedKVError):
        m.append_token(99, 1)
    s2 = m.add_sequence([1])
    m.allocate(s2, m.can_allocate(s2))
    with pytest.raises(B.PagedKVError):
        m.remove_sequence(s2)                             # table not empty
    with pytest.raises(B.PagedKVError):
        m.set_scheduled(s2, 2)                            # more than its length
    m.deallocate(s2)
    m.remove_sequence(s2)
    with pytest.raises(B.PagedKVError):
        m.block_table(s2)


# ------------------------------------------------------------------ planted mistakes
def _pin_battery():
    """Run the oracle pins above; return how many fail."""
    fails = 0
    for t in (test_oracle_prefix_hit_shares_and_revives_blocks,
              test_oracle_last_block_is_never_a_hit_and_needs_free_blocks,
              test_oracle_handing_out_a_freed_block_evicts_its_hash,
              test_oracle_token_check_guards_the_hash_index,
              test_oracle_growth_rule_at_block_boundaries,
              test_oracle_seal_chains_from_the_previous_block_across_steps,
              test_oracle_free_hits_need_free_blocks):
        try:
            t()
        except (AssertionError, KeyError, IndexError, ValueError):
            fails += 1
    return fails


def test_oracle_free_hits_need_free_blocks():
    # a hit on a free block still takes that block off the free list, so it counts
    # against the free blocks a sequence needs
    m = BlockManagerOracle(4, 4)
    a = SeqState(range(9))                      # blocks [0..3] [4..7] [8]
    m.admit(a, m.probe(a))
    _prefill_all(m, a)
    m.retire(a)                                 # all free again, two of them sealed
    x = SeqState(range(100, 105))               # takes 2 blocks off the front
    m.admit(x, m.probe(x))
    assert len(m.fifo) == 2
    b = SeqState(list(range(8)) + [50, 51, 52, 53, 54])  # 2 free hits + 2 new = 4 > 2
    assert m.probe(b) == -1


def _mutant(kind):
    class Mutant(BlockManagerOracle):
        pass
    if kind == "release_to_front":
        def _push_free(self, bid):
            self.in_use.discard(bid)
            self.fifo.appendleft(bid)
        Mutant._push_free = _push_free
    elif kind == "unchained_hash":
        import oracle.block_manager as OB
        def seal(self, s):
            first, last = s.num_cached // self.bs, (s.num_cached + s.num_scheduled) // self.bs
            for i in range(first, last):
                toks = s.block_tokens(i, self.bs)
                h = OB.block_hash(toks)             # the chain dropped
                self.seal_hash[s.table[i]] = h
                self.seal_tokens[s.table[i]] = toks
                self.index[h] = s.table[i]
        Mutant.seal = seal
    elif kind == "last_block_can_hit":
        def _hits(self, s):
            out, h = [], None
            for i in range(s.nblocks(self.bs)):    # walks the last block too
                toks = s.block_tokens(i, self.bs)
                h = block_hash(toks, h)
                bid = self.index.get(h)
                if bid is None or self.seal_tokens[bid] != toks:
                    break
                out.append(bid)
            return out
        Mutant._hits = _hits
    elif kind == "free_hits_cost_nothing":
        def probe(self, s):
            hits = self._hits(s)
            need = s.nblocks(self.bs) - len(hits)
            return -1 if len(self.fifo) < need else len(hits)
        Mutant.probe = probe
    elif kind == "grow_on_full_block":
        def grow(self, s):
            if len(s.tokens) % self.bs == 0:
                s.table.append(self._pop_free())
        def room_to_grow(self, s):
            return len(self.fifo) >= (1 if len(s.tokens) % self.bs == 0 else 0)
        Mutant.grow = grow
        Mutant.room_to_grow = room_to_grow
    elif kind == "reuse_keeps_hash":
        def _pop_free(self):
            bid = self.fifo.popleft()
            self.refs[bid] = 1
            self.in_use.add(bid)
            return bid
        Mutant._pop_free = _pop_free
    elif kind == "no_token_check":
        def _hits(self, s):
            out, h = [], None
            for i in range(s.nblocks(self.bs) - 1):
                h = block_hash(s.block_tokens(i, self.bs), h)
                bid = self.index.get(h)
                if bid is None:
                    break
                out.append(bid)
            return out
        Mutant._hits = _hits
    return Mutant


@pytest.mark.parametrize("kind", ["release_to_front", "unchained_hash", "last_block_can_hit",
                                  "free_hits_cost_nothing", "grow_on_full_block",
                                  "reuse_keeps_hash", "no_token_check"])
def test_planted_mistake_in_the_block_manager_oracle_is_caught(kind, monkeypatch):
    assert _pin_battery() == 0
    monkeypatch.setitem(globals(), "BlockManagerOracle", _mutant(kind))
    assert _pin_battery() >= 1, kind
