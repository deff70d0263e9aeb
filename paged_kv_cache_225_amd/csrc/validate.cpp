// Checks of the data-dependent preconditions of the attention and store calls.
//
// The engine in "vLLM 学习笔记 02：nano-vllm 源码逐段精读" asserts its tensor shapes in the
// store_kvcache wrapper before the scatter and trusts the rest of its metadata, which its
// own block manager and prepare_prefill / prepare_decode build. The library's kernels only
// bounds-check what they touch, so a wrong slot, length or block id gives wrong numbers but
// no fault. These checks name the first violation instead; they compute nothing else. Each
// takes its arrays from host memory, or copies them from the device first (synchronising
// the stream), and the device calls run them before launching when PKV_DEBUG is set.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <utility>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "paged_kv.h"
#include "validate.hpp"

namespace {

int fail(pkv_violation* first, int32_t check, int64_t index, int64_t value) {
  if (first) {
    first->check = check;
    first->reserved = 0;
    first->index = index;
    first->value = value;
  }
  return PKV_ERR_PRECONDITION;
}

void clear(pkv_violation* first) {
  if (first) memset(first, 0, sizeof(*first));
}

// The contents of an int32 array of n elements on the host: the array itself, or a copy of
// a device array made on `stream` (which is synchronised). Returns PKV_OK, PKV_ERR_INVALID
// (the stream is recording a graph: no copy can be made there) or PKV_ERR_HIP.
int host_view(const int32_t* p, int64_t n, int32_t on_device, hipStream_t stream,
              std::vector<int32_t>& buf, const int32_t** out) {
  if (!on_device || n == 0 || !p) {
    *out = p;
    return PKV_OK;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_HIP;
  }
  if (cs != hipStreamCaptureStatusNone) return PKV_ERR_INVALID;
  try {
    buf.resize((size_t)n);
  } catch (const std::bad_alloc&) {
    return PKV_ERR_INVALID;
  }
  if (hipMemcpyAsync(buf.data(), p, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_HIP;
  }
  *out = buf.data();
  return PKV_OK;
}

// Slots of a store: -1 (skip) or in [0, num_slots); non-negative slots unique. A duplicate
// is reported at the later of the two tokens, the earliest such token of the call.
int slots_ok(const int32_t* slots, int32_t n, int64_t num_slots, pkv_violation* first) {
  for (int32_t t = 0; t < n; ++t)
    if (slots[t] < -1 || (int64_t)slots[t] >= num_slots)
      return fail(first, PKV_CHECK_SLOT_RANGE, t, slots[t]);
  std::vector<std::pair<int32_t, int32_t>> order;  // (slot, token), slots >= 0
  try {
    order.reserve((size_t)n);
  } catch (const std::bad_alloc&) {
    return PKV_ERR_INVALID;
  }
  for (int32_t t = 0; t < n; ++t)
    if (slots[t] >= 0) order.emplace_back(slots[t], t);
  std::sort(order.begin(), order.end());
  int32_t dup_token = -1, dup_slot = 0;
  for (size_t i = 1; i < order.size(); ++i)
    if (order[i].first == order[i - 1].first &&
        (dup_token < 0 || order[i].second < dup_token)) {
      dup_token = order[i].second;  // the equal slot's second-earliest token
      dup_slot = order[i].first;
    }
  if (dup_token >= 0) return fail(first, PKV_CHECK_SLOT_DUPLICATE, dup_token, dup_slot);
  return PKV_OK;
}

// The table entries of sequence b that a call with n keys reads: the first ceil(n / bs).
int tables_ok(const int32_t* tables, int32_t width, int32_t b, int64_t n, int32_t bs,
              int32_t num_blocks, pkv_violation* first) {
  const int64_t used = (n + bs - 1) / bs;
  for (int64_t j = 0; j < used; ++j) {
    const int64_t at = (int64_t)b * width + j;
    if (tables[at] < 0 || tables[at] >= num_blocks)
      return fail(first, PKV_CHECK_BLOCK_RANGE, at, tables[at]);
  }
  return PKV_OK;
}

bool pow2_at_least_16(int32_t v) { return v >= 16 && (v & (v - 1)) == 0; }

}  // namespace

namespace pkv {

bool debug_checks_enabled() {
  static const bool on = [] {
    const char* env = getenv("PKV_DEBUG");
    return env && env[0] && strcmp(env, "0") != 0;
  }();
  return on;
}

bool run_debug_checks(hipStream_t stream) {
  if (!debug_checks_enabled()) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;  // the check's own copy then reports the failure
  }
  return cs == hipStreamCaptureStatusNone;
}

}  // namespace pkv

extern "C" {

int pkv_check_store(const int32_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                    int32_t on_device, hipStream_t stream, pkv_violation* first) {
  clear(first);
  if (num_tokens < 0 || num_slots < 0) return PKV_ERR_INVALID;
  if (num_tokens == 0) return PKV_OK;
  if (!slot_mapping) return PKV_ERR_INVALID;
  std::vector<int32_t> buf;
  const int32_t* s = nullptr;
  int rc = host_view(slot_mapping, num_tokens, on_device, stream, buf, &s);
  if (rc != PKV_OK) return rc;
  return slots_ok(s, num_tokens, num_slots, first);
}

int pkv_check_decode(const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* slot_mapping, int32_t num_seqs,
                     int32_t num_blocks, int32_t block_size, int32_t on_device,
                     hipStream_t stream, pkv_violation* first) {
  clear(first);
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks < 0) return PKV_ERR_INVALID;
  if (!pow2_at_least_16(block_size)) return PKV_ERR_INVALID;
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens) return PKV_ERR_INVALID;
  std::vector<int32_t> tb, cb, sb;
  const int32_t *t = nullptr, *c = nullptr, *s = nullptr;
  int rc = host_view(context_lens, num_seqs, on_device, stream, cb, &c);
  if (rc == PKV_OK)
    rc = host_view(block_tables, (int64_t)num_seqs * max_blocks_per_seq, on_device, stream, tb, &t);
  if (rc == PKV_OK && slot_mapping) rc = host_view(slot_mapping, num_seqs, on_device, stream, sb, &s);
  if (rc != PKV_OK) return rc;
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t n = c[b];
    if (n < 0 || n > cap) return fail(first, PKV_CHECK_CONTEXT_RANGE, b, n);
    rc = tables_ok(t, max_blocks_per_seq, b, n, block_size, num_blocks, first);
    if (rc != PKV_OK) return rc;
  }
  if (s) {
    rc = slots_ok(s, num_seqs, num_slots, first);
    if (rc != PKV_OK) return rc;
    // the newest token's slot is that of position n - 1 of its own table; a sequence
    // without keys (a padded row) stores nothing
    for (int32_t b = 0; b < num_seqs; ++b) {
      const int64_t n = c[b];
      if (s[b] == -1) continue;
      if (n == 0) return fail(first, PKV_CHECK_NEW_TOKEN_SLOT, b, s[b]);
      const int64_t pos = n - 1;
      const int64_t want = (int64_t)t[(int64_t)b * max_blocks_per_seq + pos / block_size] *
                               block_size + pos % block_size;
      if (s[b] != want) return fail(first, PKV_CHECK_NEW_TOKEN_SLOT, b, s[b]);
    }
  }
  return PKV_OK;
}

int pkv_check_prefill(const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                      int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                      int32_t max_seqlen_k, int32_t num_blocks, int32_t block_size,
                      int32_t on_device, hipStream_t stream, pkv_violation* first) {
  clear(first);
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return PKV_ERR_INVALID;
  const bool paged = block_tables != nullptr;
  if (paged && (max_blocks_per_seq <= 0 || num_blocks < 0 || !pow2_at_least_16(block_size)))
    return PKV_ERR_INVALID;
  if (num_seqs == 0) return total_q == 0 ? PKV_OK : fail(first, PKV_CHECK_CU_SEQLENS, 0, total_q);
  if (!cu_seqlens_q || !cu_seqlens_k) return PKV_ERR_INVALID;
  std::vector<int32_t> qb, kb, tb;
  const int32_t *cq = nullptr, *ck = nullptr, *t = nullptr;
  int rc = host_view(cu_seqlens_q, (int64_t)num_seqs + 1, on_device, stream, qb, &cq);
  if (rc == PKV_OK) rc = host_view(cu_seqlens_k, (int64_t)num_seqs + 1, on_device, stream, kb, &ck);
  if (rc == PKV_OK && paged)
    rc = host_view(block_tables, (int64_t)num_seqs * max_blocks_per_seq, on_device, stream, tb, &t);
  if (rc != PKV_OK) return rc;
  if (cq[0] != 0) return fail(first, PKV_CHECK_CU_SEQLENS, 0, cq[0]);
  if (ck[0] < 0) return fail(first, PKV_CHECK_CU_SEQLENS, 0, ck[0]);
  const int64_t cap = paged ? (int64_t)max_blocks_per_seq * block_size : INT64_MAX;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t lq = (int64_t)cq[b + 1] - cq[b], lk = (int64_t)ck[b + 1] - ck[b];
    if (lq < 0) return fail(first, PKV_CHECK_CU_SEQLENS, b + 1, cq[b + 1]);
    if (lk < 0) return fail(first, PKV_CHECK_CU_SEQLENS, b + 1, ck[b + 1]);
    if (lk < lq) return fail(first, PKV_CHECK_LK_LT_LQ, b, lk);
    if (lq > max_seqlen_q || lk > max_seqlen_k) return fail(first, PKV_CHECK_MAX_SEQLEN, b, lq > max_seqlen_q ? lq : lk);
    if (lk > cap) return fail(first, PKV_CHECK_CONTEXT_RANGE, b, lk);
    if (paged) {
      rc = tables_ok(t, max_blocks_per_seq, b, lk, block_size, num_blocks, first);
      if (rc != PKV_OK) return rc;
    }
  }
  if (cq[num_seqs] != total_q) return fail(first, PKV_CHECK_CU_SEQLENS, num_seqs, cq[num_seqs]);
  return PKV_OK;
}


// The groups of a shared-prefix decode call. Every entry of group_members is a pair
// (sequence, column group_col[g]); these pairs must be exactly the pairs (b, c) with
// c < shared_cols[b], each once, and the members of a group must hold one block id in
// their column (a prefix cache reuses a block only in the column its tokens occupy).
int pkv_check_prefix(const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                     const int32_t* shared_cols, const int32_t* group_ptr,
                     const int32_t* group_members, const int32_t* group_col, int32_t num_groups,
                     int32_t max_group_size, int32_t on_device, hipStream_t stream,
                     pkv_violation* first) {
  clear(first);
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_groups < 0 || max_group_size < 0)
    return PKV_ERR_INVALID;
  if (!pow2_at_least_16(block_size)) return PKV_ERR_INVALID;
  if (num_seqs > 0 && (!block_tables || !context_lens || !shared_cols)) return PKV_ERR_INVALID;
  if (num_groups > 0 && (!group_ptr || !group_col)) return PKV_ERR_INVALID;
  const int32_t W = max_blocks_per_seq;
  std::vector<int32_t> tb, cb, sb, pb, mb, gb;
  const int32_t *t = nullptr, *c = nullptr, *sc = nullptr, *ptr = nullptr, *mem = nullptr,
                *col = nullptr;
  int rc = host_view(context_lens, num_seqs, on_device, stream, cb, &c);
  if (rc == PKV_OK) rc = host_view(shared_cols, num_seqs, on_device, stream, sb, &sc);
  if (rc == PKV_OK) rc = host_view(block_tables, (int64_t)num_seqs * W, on_device, stream, tb, &t);
  if (rc == PKV_OK && num_groups > 0)
    rc = host_view(group_ptr, (int64_t)num_groups + 1, on_device, stream, pb, &ptr);
  if (rc == PKV_OK && num_groups > 0) rc = host_view(group_col, num_groups, on_device, stream, gb, &col);
  if (rc != PKV_OK) return rc;
  // shared columns: whole blocks before the newest token's, inside the table
  int64_t pairs = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t s = sc[b];
    if (s < 0 || s > W || (s > 0 && s * block_size > (int64_t)c[b] - 1))
      return fail(first, PKV_CHECK_SHARED_COLS, b, s);
    pairs += s;
  }
  int64_t total = 0;
  if (num_groups > 0) {
    if (ptr[0] != 0) return fail(first, PKV_CHECK_GROUP_PTR, 0, ptr[0]);
    for (int32_t g = 0; g < num_groups; ++g) {
      const int64_t size = (int64_t)ptr[g + 1] - ptr[g];
      if (size < 0 || size > max_group_size || ptr[g + 1] > pairs)
        return fail(first, PKV_CHECK_GROUP_PTR, (int64_t)g + 1, ptr[g + 1]);
      if (col[g] < 0 || col[g] >= W) return fail(first, PKV_CHECK_GROUP_COL, g, col[g]);
    }
    total = ptr[num_groups];
  }
  if (total != pairs) return fail(first, PKV_CHECK_GROUP_PTR, num_groups, total);
  if (total == 0) return PKV_OK;
  if (!group_members) return PKV_ERR_INVALID;
  rc = host_view(group_members, total, on_device, stream, mb, &mem);
  if (rc != PKV_OK) return rc;
  // pair (b, c) -> seen; as many pairs as entries, so a repeat or a pair outside the
  // shared columns is found at the entry that makes it
  std::vector<int64_t> base;
  std::vector<uint8_t> seen;
  try {
    base.resize((size_t)num_seqs + 1);
    seen.assign((size_t)pairs, 0);
  } catch (const std::bad_alloc&) {
    return PKV_ERR_INVALID;
  }
  base[0] = 0;
  for (int32_t b = 0; b < num_seqs; ++b) base[b + 1] = base[b] + sc[b];
  for (int32_t g = 0; g < num_groups; ++g) {
    int32_t block = 0;
    for (int64_t e = ptr[g]; e < ptr[g + 1]; ++e) {
      const int32_t b = mem[e];
      if (b < 0 || b >= num_seqs) return fail(first, PKV_CHECK_GROUP_MEMBER, e, b);
      if (col[g] >= sc[b] || seen[base[b] + col[g]]) return fail(first, PKV_CHECK_PREFIX_COVER, b, col[g]);
      seen[base[b] + col[g]] = 1;
      const int32_t id = t[(int64_t)b * W + col[g]];
      if (e == ptr[g]) block = id;
      else if (id != block) return fail(first, PKV_CHECK_GROUP_BLOCK, e, id);
    }
  }
  return PKV_OK;  // pairs entries, none repeated: every shared pair is covered
}

}  // extern "C"
