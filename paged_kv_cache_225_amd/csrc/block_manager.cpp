// Host block manager of the paged KV cache with prefix caching.
//
// "vLLM 学习笔记 02：nano-vllm 源码逐段精读" (the Block, BlockManager and Sequence listings,
// and the Scheduler that drives them) describes the policy this file implements:
//   - The pool is num_blocks blocks of block_size token slots. A block is free (on a FIFO of
//     free ids) or used (reference count >= 1, one count per sequence whose table holds it).
//   - A full block that has been computed is sealed: it records its token ids and a hash
//     chained over the whole prefix (the previous block's hash, as 8 little-endian bytes,
//     followed by this block's token ids as 64-bit little-endian integers, through XXH64 with
//     seed 0), and the hash maps to the block in an index.
//   - Admitting a sequence first walks its full blocks except the last: each one whose
//     chained hash is in the index with equal token ids is a cache hit, until the first
//     miss. Hits reuse the indexed block (a used one gains a reference, a free one is taken
//     off the free FIFO wherever it sits); the other blocks come from the front of the FIFO.
//     A block taken from the FIFO loses its index entry (if the index still points at it)
//     and its sealed contents. The admission check refuses when the FIFO holds fewer blocks
//     than the sequence needs beyond its hits on blocks that are in use.
//   - Retiring a sequence drops one reference per table entry, last entry first; a block
//     reaching zero goes to the back of the FIFO but keeps its seal, so a later admission
//     can still hit it until it is handed out again.
//   - Decode grows a table by one block when the sequence's length is one past a multiple
//     of block_size (the new token starts a block), and may only proceed when the FIFO can
//     supply it.
//   - After a step, the blocks completed by the step's tokens are sealed, chaining from the
//     previous block's hash.
// XXH64 follows its published specification (Yann Collet, xxHash, "XXH64 algorithm").
#include <stdint.h>
#include <string.h>

#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "paged_kv.h"

namespace {

// ---------------------------------------------------------------- XXH64
constexpr uint64_t kP1 = 0x9E3779B185EBCA87ULL;
constexpr uint64_t kP2 = 0xC2B2AE3D27D4EB4FULL;
constexpr uint64_t kP3 = 0x165667B19E3779F9ULL;
constexpr uint64_t kP4 = 0x85EBCA77C2B2AE63ULL;
constexpr uint64_t kP5 = 0x27D4EB2F165667C5ULL;

inline uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
inline uint64_t rd64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];  // little-endian, any alignment
  return v;
}
inline uint32_t rd32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
inline uint64_t lane_round(uint64_t acc, uint64_t in) { return rotl(acc + in * kP2, 31) * kP1; }
inline uint64_t merge_lane(uint64_t h, uint64_t v) { return (h ^ lane_round(0, v)) * kP1 + kP4; }

uint64_t xxh64(const uint8_t* p, size_t n, uint64_t seed) {
  const uint8_t* end = p + n;
  uint64_t h;
  if (n >= 32) {
    uint64_t v[4] = {seed + kP1 + kP2, seed + kP2, seed, seed - kP1};
    for (; end - p >= 32; p += 32)
      for (int i = 0; i < 4; ++i) v[i] = lane_round(v[i], rd64(p + 8 * i));
    h = rotl(v[0], 1) + rotl(v[1], 7) + rotl(v[2], 12) + rotl(v[3], 18);
    for (int i = 0; i < 4; ++i) h = merge_lane(h, v[i]);
  } else {
    h = seed + kP5;
  }
  h += (uint64_t)n;
  for (; end - p >= 8; p += 8) h = rotl(h ^ lane_round(0, rd64(p)), 27) * kP1 + kP4;
  if (end - p >= 4) {
    h = rotl(h ^ ((uint64_t)rd32(p) * kP1), 23) * kP2 + kP3;
    p += 4;
  }
  for (; p < end; ++p) h = rotl(h ^ ((uint64_t)*p * kP5), 11) * kP1;
  h ^= h >> 33;
  h *= kP2;
  h ^= h >> 29;
  h *= kP3;
  h ^= h >> 32;
  return h;
}

// The chained hash of one block: [prefix as 8 LE bytes, if any] + token ids as int64 LE.
uint64_t block_hash(const int64_t* tokens, int64_t n, bool has_prefix, uint64_t prefix) {
  std::vector<uint8_t> buf;
  buf.reserve((size_t)(n + 1) * 8);
  auto put = [&](uint64_t v) {
    for (int i = 0; i < 8; ++i) buf.push_back((uint8_t)(v >> (8 * i)));
  };
  if (has_prefix) put(prefix);
  for (int64_t i = 0; i < n; ++i) put((uint64_t)tokens[i]);
  return xxh64(buf.data(), buf.size(), 0);
}

struct Block {
  int32_t refs = 0;
  bool sealed = false;  // carries a hash and its token ids
  uint64_t hash = 0;
  std::vector<int64_t> tokens;
};

struct Seq {
  std::vector<int64_t> tokens;
  std::vector<int32_t> table;
  int64_t num_cached = 0;
  int64_t num_scheduled = 0;
  bool live = true;
};

}  // namespace

struct pkv_block_manager {
  int32_t block_size = 0;
  std::vector<Block> blocks;
  std::unordered_map<uint64_t, int32_t> index;  // sealed hash -> block id
  std::deque<int32_t> free_ids;
  std::unordered_set<int32_t> used;
  std::vector<Seq> seqs;

  int64_t num_blocks_of(const Seq& s) const {
    return ((int64_t)s.tokens.size() + block_size - 1) / block_size;
  }
  const int64_t* block_tokens(const Seq& s, int64_t i, int64_t* n) const {
    const int64_t lo = i * block_size;
    const int64_t hi = lo + block_size < (int64_t)s.tokens.size() ? lo + block_size : (int64_t)s.tokens.size();
    *n = hi - lo;
    return s.tokens.data() + lo;
  }
  // walks the leading full blocks (all but the last block) while they are cache hits
  template <typename F>
  int64_t walk_hits(const Seq& s, F&& on_hit) const {
    bool has = false;
    uint64_t h = 0;
    int64_t hits = 0;
    for (int64_t i = 0; i + 1 < num_blocks_of(s); ++i) {
      int64_t n;
      const int64_t* t = block_tokens(s, i, &n);
      h = block_hash(t, n, has, h);
      has = true;
      auto it = index.find(h);
      if (it == index.end()) break;
      const Block& b = blocks[it->second];
      if ((int64_t)b.tokens.size() != n || memcmp(b.tokens.data(), t, (size_t)n * 8) != 0) break;
      on_hit(it->second);
      ++hits;
    }
    return hits;
  }
  int32_t take_free() {
    const int32_t id = free_ids.front();
    free_ids.pop_front();
    Block& b = blocks[id];
    if (b.sealed) {
      auto it = index.find(b.hash);
      if (it != index.end() && it->second == id) index.erase(it);
    }
    b.refs = 1;
    b.sealed = false;
    b.hash = 0;
    b.tokens.clear();
    used.insert(id);
    return id;
  }
  void release(int32_t id) {
    used.erase(id);
    free_ids.push_back(id);
  }
  Seq* seq(int32_t id) {
    if (id < 0 || id >= (int32_t)seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
};

extern "C" {

uint64_t pkv_xxh64(const void* data, size_t len, uint64_t seed) {
  return xxh64(static_cast<const uint8_t*>(data), data ? len : 0, seed);
}

int pkv_block_hash(const int64_t* token_ids, int32_t num_tokens, int32_t has_prefix,
                   uint64_t prefix, uint64_t* hash_out) {
  if (!hash_out || num_tokens < 0 || (num_tokens > 0 && !token_ids)) return PKV_ERR_INVALID;
  *hash_out = block_hash(token_ids, num_tokens, has_prefix != 0, prefix);
  return PKV_OK;
}

int pkv_bm_create(pkv_block_manager** handle, int32_t num_blocks, int32_t block_size) {
  if (!handle) return PKV_ERR_INVALID;
  *handle = nullptr;
  if (num_blocks < 1 || block_size < 2) return PKV_ERR_INVALID;
  pkv_block_manager* m = new (std::nothrow) pkv_block_manager;
  if (!m) return PKV_ERR_INVALID;
  m->block_size = block_size;
  m->blocks.resize((size_t)num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) m->free_ids.push_back(i);
  *handle = m;
  return PKV_OK;
}

int pkv_bm_destroy(pkv_block_manager* m) {
  if (!m) return PKV_ERR_INVALID;
  delete m;
  return PKV_OK;
}

int pkv_bm_add_sequence(pkv_block_manager* m, const int64_t* token_ids, int32_t num_tokens) {
  if (!m || num_tokens < 1 || !token_ids) return PKV_ERR_INVALID;
  Seq s;
  s.tokens.assign(token_ids, token_ids + num_tokens);
  m->seqs.push_back(std::move(s));
  return (int)m->seqs.size() - 1;
}

int pkv_bm_append_token(pkv_block_manager* m, int32_t seq, int64_t token_id) {
  Seq* s = m ? m->seq(seq) : nullptr;
  if (!s) return PKV_ERR_INVALID;
  s->tokens.push_back(token_id);
  return PKV_OK;
}

int pkv_bm_can_allocate(const pkv_block_manager* m, int32_t seq) {
  if (!m) return PKV_ERR_INVALID;
  auto* mm = const_cast<pkv_block_manager*>(m);
  Seq* s = mm->seq(seq);
  if (!s || !s->table.empty()) return PKV_ERR_INVALID;
  int64_t need = m->num_blocks_of(*s);
  const int64_t hits = m->walk_hits(*s, [&](int32_t id) {
    if (m->used.count(id)) --need;  // shared with a running sequence: no new block
  });
  return (int64_t)m->free_ids.size() < need ? -1 : (int)hits;
}

int pkv_bm_allocate(pkv_block_manager* m, int32_t seq, int32_t num_cached_blocks) {
  Seq* s = m ? m->seq(seq) : nullptr;
  if (!s || !s->table.empty() || num_cached_blocks < 0) return PKV_ERR_INVALID;
  const int64_t nb = m->num_blocks_of(*s);
  // the hits must still be hits, and the free list must cover the rest
  std::vector<int32_t> hit_ids;
  m->walk_hits(*s, [&](int32_t id) {
    if ((int32_t)hit_ids.size() < num_cached_blocks) hit_ids.push_back(id);
  });
  if ((int32_t)hit_ids.size() < num_cached_blocks) return PKV_ERR_INVALID;
  int64_t from_free = nb - num_cached_blocks;
  for (int32_t id : hit_ids)
    if (!m->used.count(id)) ++from_free;  // a free hit leaves the FIFO too
  if ((int64_t)m->free_ids.size() < from_free) return PKV_ERR_INVALID;
  for (int32_t id : hit_ids) {
    Block& b = m->blocks[id];
    if (m->used.count(id)) {
      ++b.refs;
    } else {
      b.refs = 1;
      for (auto it = m->free_ids.begin(); it != m->free_ids.end(); ++it)
        if (*it == id) {
          m->free_ids.erase(it);
          break;
        }
      m->used.insert(id);
    }
    s->table.push_back(id);
  }
  for (int64_t i = num_cached_blocks; i < nb; ++i) s->table.push_back(m->take_free());
  s->num_cached = (int64_t)num_cached_blocks * m->block_size;
  return PKV_OK;
}

int pkv_bm_deallocate(pkv_block_manager* m, int32_t seq) {
  Seq* s = m ? m->seq(seq) : nullptr;
  if (!s) return PKV_ERR_INVALID;
  for (auto it = s->table.rbegin(); it != s->table.rend(); ++it) {
    Block& b = m->blocks[*it];
    if (--b.refs == 0) m->release(*it);
  }
  s->table.clear();
  s->num_cached = 0;
  s->num_scheduled = 0;
  return PKV_OK;
}

int pkv_bm_can_append(const pkv_block_manager* m, int32_t seq) {
  if (!m) return PKV_ERR_INVALID;
  Seq* s = const_cast<pkv_block_manager*>(m)->seq(seq);
  if (!s) return PKV_ERR_INVALID;
  const bool starts_block = (int64_t)s->tokens.size() % m->block_size == 1;
  return (int64_t)m->free_ids.size() >= (starts_block ? 1 : 0) ? 1 : 0;
}

int pkv_bm_may_append(pkv_block_manager* m, int32_t seq) {
  Seq* s = m ? m->seq(seq) : nullptr;
  if (!s) return PKV_ERR_INVALID;
  const bool starts_block = (int64_t)s->tokens.size() % m->block_size == 1;
  if (starts_block) {
    if (m->free_ids.empty()) return PKV_ERR_INVALID;
    s->table.push_back(m->take_free());
  }
  return PKV_OK;
}

int pkv_bm_set_scheduled(pkv_block_manager* m, int32_t seq, int32_t num_scheduled_tokens) {
  Seq* s = m ? m->seq(seq) : nullptr;
  if (!s || num_scheduled_tokens < 0 ||
      s->num_cached + num_scheduled_tokens > (int64_t)s->tokens.size())
    return PKV_ERR_INVALID;
  s->num_scheduled = num_scheduled_tokens;
  return PKV_OK;
}

int pkv_bm_hash_blocks(pkv_block_manager* m, int32_t seq) {
  Seq* s = m ? m->seq(seq) : nullptr;
  if (!s) return PKV_ERR_INVALID;
  const int64_t start = s->num_cached / m->block_size;
  const int64_t end = (s->num_cached + s->num_scheduled) / m->block_size;
  if (end > (int64_t)s->table.size()) return PKV_ERR_INVALID;
  bool has = false;
  uint64_t h = 0;
  if (start > 0 && start < end) {
    const Block& prev = m->blocks[s->table[start - 1]];
    has = prev.sealed;
    h = prev.hash;
  }
  for (int64_t i = start; i < end; ++i) {
    int64_t n;
    const int64_t* t = m->block_tokens(*s, i, &n);
    h = block_hash(t, n, has, h);
    has = true;
    const int32_t id = s->table[i];
    Block& b = m->blocks[id];
    b.sealed = true;
    b.hash = h;
    b.tokens.assign(t, t + n);
    m->index[h] = id;
  }
  return PKV_OK;
}

int pkv_bm_commit_scheduled(pkv_block_manager* m, int32_t seq) {
  Seq* s = m ? m->seq(seq) : nullptr;
  if (!s) return PKV_ERR_INVALID;
  s->num_cached += s->num_scheduled;
  s->num_scheduled = 0;
  return PKV_OK;
}

int pkv_bm_sequence_info(const pkv_block_manager* m, int32_t seq, int64_t* num_tokens,
                         int64_t* num_cached_tokens, int64_t* num_scheduled_tokens,
                         int32_t* table_len) {
  if (!m) return PKV_ERR_INVALID;
  Seq* s = const_cast<pkv_block_manager*>(m)->seq(seq);
  if (!s) return PKV_ERR_INVALID;
  if (num_tokens) *num_tokens = (int64_t)s->tokens.size();
  if (num_cached_tokens) *num_cached_tokens = s->num_cached;
  if (num_scheduled_tokens) *num_scheduled_tokens = s->num_scheduled;
  if (table_len) *table_len = (int32_t)s->table.size();
  return PKV_OK;
}

int pkv_bm_block_table(const pkv_block_manager* m, int32_t seq, int32_t* out, int32_t capacity) {
  if (!m || capacity < 0 || (capacity > 0 && !out)) return PKV_ERR_INVALID;
  Seq* s = const_cast<pkv_block_manager*>(m)->seq(seq);
  if (!s) return PKV_ERR_INVALID;
  const int n = (int)s->table.size();
  for (int i = 0; i < n && i < capacity; ++i) out[i] = s->table[i];
  return n;
}

int pkv_bm_num_free_blocks(const pkv_block_manager* m) {
  return m ? (int)m->free_ids.size() : PKV_ERR_INVALID;
}

int pkv_bm_free_block_ids(const pkv_block_manager* m, int32_t* out, int32_t capacity) {
  if (!m || capacity < 0 || (capacity > 0 && !out)) return PKV_ERR_INVALID;
  const int n = (int)m->free_ids.size();
  int i = 0;
  for (auto it = m->free_ids.begin(); it != m->free_ids.end() && i < capacity; ++it) out[i++] = *it;
  return n;
}

int pkv_bm_block_info(const pkv_block_manager* m, int32_t block_id, int32_t* ref_count,
                      int32_t* sealed, uint64_t* hash) {
  if (!m || block_id < 0 || block_id >= (int32_t)m->blocks.size()) return PKV_ERR_INVALID;
  const Block& b = m->blocks[block_id];
  if (ref_count) *ref_count = b.refs;
  if (sealed) *sealed = b.sealed ? 1 : 0;
  if (hash) *hash = b.hash;
  return PKV_OK;
}

int pkv_bm_remove_sequence(pkv_block_manager* m, int32_t seq) {
  Seq* s = m ? m->seq(seq) : nullptr;
  if (!s || !s->table.empty()) return PKV_ERR_INVALID;
  s->live = false;
  s->tokens.clear();
  s->tokens.shrink_to_fit();
  return PKV_OK;
}

}  // extern "C"
