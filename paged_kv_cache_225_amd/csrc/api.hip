// C ABI of the paged-attention library: argument validation, host metadata, launches.
// The operations and their sources are documented in include/paged_kv.h.
#include <limits.h>
#include <stdlib.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "paged_kv.h"
#include "validate.hpp"

// The decode workspace of paged_attn_decode_noalloc: device memory that the library owns, so
// that a caller who cannot allocate (graph capture, a serving loop that forbids allocation)
// passes inputs and outputs only. Each GPU the library runs on holds its own copy of the
// array from module load until the process ends. Host code never passes `scratch` itself
// (on the host its name stands for a host-side shadow, not a device address): it asks the
// runtime for the device address once per device and passes that.
static __device__ __align__(256) char scratch[PKV_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 256;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, looked up on the first call on that
// device (with it current) and kept for the process.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    return PKV_ERR_HIP;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return PKV_ERR_HIP;
      }
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKV_OK;
}

bool pow2_at_least_16(int32_t v) { return v >= 16 && (v & (v - 1)) == 0; }
bool supported_group(int32_t heads, int32_t kv_heads) {
  if (heads <= 0 || kv_heads <= 0 || heads % kv_heads) return false;
  const int32_t g = heads / kv_heads;
  return g == 1 || g == 2 || g == 4 || g == 8;
}
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Cap of the decode grid: PKV_DECODE_WORKGROUPS if set to a positive integer when the
// library first launches a decode call, else the built-in default. Read once; a tuning knob
// that changes how the keys are split, never what is computed.
int32_t decode_workgroups() {
  static const int32_t v = [] {
    const char* env = getenv("PKV_DECODE_WORKGROUPS");
    const int n = env ? atoi(env) : 0;
    return n > 0 ? (int32_t)n : (int32_t)pkv::kDecodeDefaultWorkgroups;
  }();
  return v;
}

// The attention kernels move rows in 16-byte vector accesses.
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// The library's smallest share when the caller passes 0: finer when the call can hold little
// work (num_seqs * cap keys at most), so that a small batch still spreads over many
// workgroups - a share of 256 keys leaves a batch-1 step streaming through a few of them.
constexpr int64_t kFineShareKeys = 65536;     // below: 64-key shares
constexpr int64_t kMediumShareKeys = 131072;  // up to: 128-key shares; above: the default
int32_t default_partition(int64_t num_seqs, int64_t cap) {
  const int64_t upper = num_seqs * cap;
  if (upper < kFineShareKeys) return 64;
  if (upper <= kMediumShareKeys) return 128;
  return pkv::kDecodeDefaultPartition;
}

int decode_parts(int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                 int32_t partition, int32_t* part_out, int64_t* max_parts_out) {
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  if (cap > INT32_MAX) return PKV_ERR_INVALID;
  const int32_t part = partition == 0 ? default_partition(num_seqs, cap) : partition;
  if (part < 64 || part > pkv::kDecodeMaxPartition || part % 64) return PKV_ERR_INVALID;
  *part_out = part;
  *max_parts_out = ceil_div(cap, part) + 1;  // pieces a segment can be cut into
  return PKV_OK;
}

// Bytes of the partial slots and split metadata of one call.
size_t decode_ws_bytes(int64_t num_seqs, int64_t num_heads, int64_t head_dim, int64_t max_parts) {
  return (size_t)num_seqs * num_heads * max_parts * (head_dim + 2) * sizeof(float) +
         ((size_t)num_seqs + 2) * sizeof(int32_t);
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_HIP: return "HIP launch error";
    case PKV_ERR_PRECONDITION: return "data-dependent precondition violated";
    default: return "unknown status";
  }
}

// ------------------------------------------------------------------------- host metadata
int pkv_prefill_metadata(int32_t num_seqs, const int32_t* num_cached, const int32_t* num_scheduled,
                         const int32_t* block_table_flat, const int64_t* block_table_offsets,
                         int32_t block_size, int32_t table_width,
                         int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                         int32_t* max_seqlen_q, int32_t* max_seqlen_k,
                         int32_t* slot_mapping, int64_t slot_capacity, int64_t* positions,
                         int32_t* block_tables) {
  if (num_seqs < 0 || block_size <= 0 || table_width < 0 || slot_capacity < 0) return PKV_ERR_INVALID;
  if (!cu_seqlens_q || !cu_seqlens_k || !max_seqlen_q || !max_seqlen_k) return PKV_ERR_INVALID;
  if (num_seqs > 0 && (!num_cached || !num_scheduled || !block_table_offsets)) return PKV_ERR_INVALID;
  // validation pass: nothing is written on error
  int64_t total_q = 0, total_k = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t start = num_cached[b], sched = num_scheduled[b];
    const int64_t have = block_table_offsets[b + 1] - block_table_offsets[b];
    if (start < 0 || sched < 0 || have < 0 || have > table_width) return PKV_ERR_INVALID;
    const int64_t end = start + sched;
    if (have < ceil_div(end, block_size)) return PKV_ERR_INVALID;
    if (have > 0 && !block_table_flat) return PKV_ERR_INVALID;
    total_q += sched;
    total_k += end;
    for (int64_t i = 0; i < have; ++i) {
      const int64_t id = block_table_flat[block_table_offsets[b] + i];
      if (id < 0 || (id + 1) * (int64_t)block_size - 1 > INT32_MAX) return PKV_ERR_INVALID;
    }
  }
  if (total_q > INT32_MAX || total_k > INT32_MAX) return PKV_ERR_INVALID;
  if (slot_capacity > 0 && total_q > slot_capacity) return PKV_ERR_INVALID;  // 0: unchecked
  if (total_q > 0 && !slot_mapping) return PKV_ERR_INVALID;
  if (num_seqs > 0 && table_width > 0 && !block_tables) return PKV_ERR_INVALID;

  int32_t mq = 0, mk = 0;
  int64_t n = 0;
  cu_seqlens_q[0] = 0;
  cu_seqlens_k[0] = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t start = num_cached[b];
    const int32_t seqlen_q = num_scheduled[b];
    const int32_t end = start + seqlen_q;  // = seqlen_k
    const int32_t* table = block_table_flat + block_table_offsets[b];
    const int64_t have = block_table_offsets[b + 1] - block_table_offsets[b];
    cu_seqlens_q[b + 1] = cu_seqlens_q[b] + seqlen_q;
    cu_seqlens_k[b + 1] = cu_seqlens_k[b] + end;
    if (seqlen_q > mq) mq = seqlen_q;
    if (end > mk) mk = end;
    // walk the blocks that overlap [start, end); each contributes a run of consecutive slots
    for (int32_t i = start / block_size; i * (int64_t)block_size < end; ++i) {
      const int32_t first_pos = i * block_size;
      const int32_t lo = start > first_pos ? start : first_pos;
      const int32_t hi = end < first_pos + block_size ? end : first_pos + block_size;
      const int32_t base = table[i] * block_size - first_pos;
      for (int32_t p = lo; p < hi; ++p, ++n) {
        slot_mapping[n] = base + p;
        if (positions) positions[n] = p;
      }
    }
    if (block_tables)
      for (int32_t i = 0; i < table_width; ++i)
        block_tables[(int64_t)b * table_width + i] = i < have ? table[i] : -1;
  }
  *max_seqlen_q = mq;
  *max_seqlen_k = mk;
  return PKV_OK;
}

int pkv_decode_metadata(int32_t num_seqs, const int32_t* seq_lens,
                        const int32_t* block_table_flat, const int64_t* block_table_offsets,
                        int32_t block_size, int32_t table_width,
                        int32_t* slot_mapping, int32_t* context_lens, int64_t* positions,
                        int32_t* block_tables) {
  if (num_seqs < 0 || block_size <= 0 || table_width < 0) return PKV_ERR_INVALID;
  if (num_seqs == 0) return PKV_OK;
  if (!seq_lens || !block_table_flat || !block_table_offsets || !slot_mapping || !context_lens)
    return PKV_ERR_INVALID;
  if (table_width > 0 && !block_tables) return PKV_ERR_INVALID;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t len = seq_lens[b];
    const int64_t have = block_table_offsets[b + 1] - block_table_offsets[b];
    if (len < 1 || have != ceil_div(len, block_size) || have > table_width) return PKV_ERR_INVALID;
    const int64_t last = block_table_flat[block_table_offsets[b + 1] - 1];
    if (last < 0 || (last + 1) * (int64_t)block_size - 1 > INT32_MAX) return PKV_ERR_INVALID;
  }
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t len = seq_lens[b];
    const int32_t* table = block_table_flat + block_table_offsets[b];
    const int32_t num_blocks = (int32_t)(block_table_offsets[b + 1] - block_table_offsets[b]);
    const int32_t last_block_num_tokens = len - (num_blocks - 1) * block_size;
    slot_mapping[b] = table[num_blocks - 1] * block_size + last_block_num_tokens - 1;
    context_lens[b] = len;
    if (positions) positions[b] = len - 1;
    for (int32_t i = 0; i < table_width; ++i)
      block_tables[(int64_t)b * table_width + i] = i < num_blocks ? table[i] : -1;
  }
  return PKV_OK;
}

// ------------------------------------------------------------------------- store
int store_kvcache(const void* key, int64_t key_token_stride, const void* value,
                  int64_t value_token_stride, void* k_cache, void* v_cache, int64_t num_slots,
                  const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                  int32_t head_dim, pkv_dtype_t dtype, hipStream_t stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_slots < 0 || num_kv_heads <= 0 || head_dim <= 0) return PKV_ERR_INVALID;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (row > INT32_MAX) return PKV_ERR_INVALID;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_INVALID;
  if (key_token_stride < row || value_token_stride < row) return PKV_ERR_INVALID;
  if (pkv::run_debug_checks(stream)) {
    const int chk = pkv_check_store(slot_mapping, num_tokens, num_slots, 1, stream, nullptr);
    if (chk != PKV_OK) return chk;
  }
  const int rc = pkv::launch_store_kvcache(key, key_token_stride, value, value_token_stride,
                                           k_cache, v_cache, num_slots, slot_mapping, num_tokens,
                                           (int32_t)row, dtype == PKV_BF16 ? 2 : 4, stream);
  return rc == 0 ? PKV_OK : PKV_ERR_HIP;
}

// ------------------------------------------------------------------------- decode
size_t paged_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                         int32_t max_blocks_per_seq, int32_t block_size,
                                         int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0)
    return 0;
  int32_t part;
  int64_t max_parts;
  if (decode_parts(num_seqs, max_blocks_per_seq, block_size, partition_size, &part, &max_parts) != PKV_OK)
    return 0;
  size_t bytes = decode_ws_bytes(num_seqs, num_heads, head_dim, max_parts);
  if (partition_size == 0) {
    // the default share shrinks for fewer sequences, so a smaller call can need more slots
    // per row: report the largest need of any call with at most num_seqs sequences, so that
    // one workspace serves them all (the decode graphs record every bucket over one)
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    for (int64_t m : {(kFineShareKeys - 1) / cap, kMediumShareKeys / cap}) {
      if (m < 1 || m >= num_seqs) continue;
      const int64_t mp = ceil_div(cap, default_partition(m, cap)) + 1;
      const size_t b = decode_ws_bytes(m, num_heads, head_dim, mp);
      if (b > bytes) bytes = b;
    }
  }
  return bytes;
}

}  // extern "C"

namespace {

// The shared leading blocks of a paged_attn_decode_prefix call (see the header).
struct SharedPrefix {
  const int32_t* cols;
  const int32_t* group_ptr;
  const int32_t* group_members;
  const int32_t* group_col;
  int32_t num_groups, max_group_size;
};

// Bytes of the shared blocks' partial slots: (D + 2) floats per (sequence, head, column).
size_t prefix_slot_bytes(int64_t num_seqs, int64_t num_heads, int64_t head_dim, int64_t width) {
  return (size_t)num_seqs * num_heads * width * (head_dim + 2) * sizeof(float);
}
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The shared body of paged_attn_decode, paged_attn_decode_store (fused) and
// paged_attn_decode_prefix (sp: the shared leading blocks).
int decode_common(void* out, const void* q, const void* k_cache, const void* v_cache,
                  int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                  pkv_dtype_t dtype, int32_t partition_size, const int32_t* kv_stream_from,
                  void* workspace, size_t workspace_bytes, bool fused, const void* key,
                  int64_t key_token_stride, const void* value, int64_t value_token_stride,
                  const int32_t* slot_mapping, bool debug_checks, hipStream_t stream,
                  const SharedPrefix* sp = nullptr) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (sp) {
    // the shared blocks go through bf16 MFMA tiles of 64 keys, addressed with 32-bit byte
    // offsets from a tile's first row
    if (dtype != PKV_BF16 || block_size < 64) return PKV_ERR_UNSUPPORTED;
    if ((int64_t)num_kv_heads * head_dim > (INT32_MAX >> 7)) return PKV_ERR_UNSUPPORTED;
    if (sp->num_groups < 0 || sp->max_group_size < 0) return PKV_ERR_INVALID;
    if (sp->num_groups > 65535 || (sp->max_group_size + 63) / 64 > 65535) return PKV_ERR_UNSUPPORTED;
  }
  if (num_seqs < 0 || num_blocks < 1 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID;
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads) return PKV_ERR_INVALID;
  if (!pow2_at_least_16(block_size)) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (!supported_group(num_heads, num_kv_heads)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs > 16383) return PKV_ERR_UNSUPPORTED;  // the context prefix lives in 64 KiB of LDS
  // the kernels number every key row of every (sequence, kv head) with an int32
  if ((int64_t)num_seqs * max_blocks_per_seq * block_size * num_kv_heads > INT32_MAX)
    return PKV_ERR_UNSUPPORTED;
  int32_t part;
  int64_t max_parts;
  if (decode_parts(num_seqs, max_blocks_per_seq, block_size, partition_size, &part, &max_parts) != PKV_OK)
    return PKV_ERR_INVALID;
  const int elem = dtype == PKV_BF16 ? 2 : 4;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (fused) {
    if (key_token_stride < row || value_token_stride < row) return PKV_ERR_INVALID;
    if ((key_token_stride * elem) % 16 || (value_token_stride * elem) % 16) return PKV_ERR_INVALID;
  }
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_INVALID;
  if (fused && (!key || !value || !slot_mapping)) return PKV_ERR_INVALID;
  if (sp && (!sp->cols || (sp->num_groups > 0 && sp->max_group_size > 0 &&
                           (!sp->group_ptr || !sp->group_members || !sp->group_col))))
    return PKV_ERR_INVALID;
  const size_t need = paged_attn_decode_workspace_bytes(num_seqs, num_heads, head_dim,
                                                        max_blocks_per_seq, block_size,
                                                        partition_size);
  const size_t need_all = sp ? align256(need) + prefix_slot_bytes(num_seqs, num_heads, head_dim,
                                                                  max_blocks_per_seq)
                             : need;
  if (!workspace || workspace_bytes < need_all) return PKV_ERR_WORKSPACE;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(workspace))
    return PKV_ERR_INVALID;
  if (fused && (!aligned16(key) || !aligned16(value))) return PKV_ERR_INVALID;
  if (debug_checks && pkv::run_debug_checks(stream)) {
    const int chk = pkv_check_decode(block_tables, max_blocks_per_seq, context_lens,
                                     fused ? slot_mapping : nullptr, num_seqs, num_blocks,
                                     block_size, 1, stream, nullptr);
    if (chk != PKV_OK) return chk;
    if (sp) {
      const int pchk = pkv_check_prefix(block_tables, max_blocks_per_seq, context_lens,
                                        num_seqs, block_size, sp->cols, sp->group_ptr,
                                        sp->group_members, sp->group_col, sp->num_groups,
                                        sp->max_group_size, 1, stream, nullptr);
      if (pchk != PKV_OK) return pchk;
    }
  }
  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.scale = scale;
  a.bf16 = dtype == PKV_BF16;
  a.partition = part;
  a.max_parts = (int32_t)max_parts;
  a.ws_o = (float*)workspace;
  a.max_workgroups = decode_workgroups();
  a.kv_stream_from = kv_stream_from;  // device [num_seqs] or null
  a.ws_ml = (float*)workspace + (size_t)num_seqs * num_heads * max_parts * head_dim;
  a.ws_meta = (int32_t*)(a.ws_ml + (size_t)num_seqs * num_heads * max_parts * 2);
  a.new_k = fused ? key : nullptr;  // the kernels key the fused path on new_k
  a.new_k_stride = key_token_stride;
  a.new_v = value;
  a.new_v_stride = value_token_stride;
  a.slot_mapping = slot_mapping;
  a.num_slots = (int64_t)num_blocks * block_size;
  a.prefix = sp ? 1 : 0;
  a.pfx = pkv::PrefixArgs{};
  if (sp) {
    a.kv_stream_from = sp->cols;  // the stream kernel skips (and the combine merges) them
    pkv::PrefixArgs& p = a.pfx;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.num_blocks = num_blocks;
    p.block_tables = block_tables;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.group_ptr = sp->group_ptr;
    p.group_members = sp->group_members;
    p.group_col = sp->group_col;
    p.num_groups = sp->num_groups;
    p.max_group_size = sp->max_group_size;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.head_dim = head_dim;
    p.block_size = block_size;
    p.scale = scale;
    p.pfx_o = (float*)((char*)workspace + align256(need));
    p.pfx_ml = p.pfx_o + (size_t)num_seqs * num_heads * max_blocks_per_seq * head_dim;
  }
  const int rc = pkv::launch_decode(a, stream);
  return rc == 0 ? PKV_OK : (rc == -2 ? PKV_ERR_UNSUPPORTED : PKV_ERR_HIP);
}

}  // namespace

extern "C" {

int paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                      pkv_dtype_t dtype, int32_t partition_size,
                      const int32_t* kv_stream_from, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return decode_common(out, q, k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       scale, dtype, partition_size, kv_stream_from, workspace, workspace_bytes,
                       false, nullptr,
                       0, nullptr, 0, nullptr, true, stream);
}

size_t paged_attn_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                                int32_t head_dim, int32_t max_blocks_per_seq,
                                                int32_t block_size, int32_t partition_size) {
  const size_t base = paged_attn_decode_workspace_bytes(num_seqs, num_heads, head_dim,
                                                        max_blocks_per_seq, block_size,
                                                        partition_size);
  if (base == 0) return 0;
  return align256(base) + prefix_slot_bytes(num_seqs, num_heads, head_dim, max_blocks_per_seq);
}

int paged_attn_decode_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                             int32_t num_blocks, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, float scale,
                             pkv_dtype_t dtype, int32_t partition_size,
                             const int32_t* shared_cols, const int32_t* group_ptr,
                             const int32_t* group_members, const int32_t* group_col,
                             int32_t num_groups, int32_t max_group_size, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  const SharedPrefix sp{shared_cols, group_ptr, group_members, group_col, num_groups,
                        max_group_size};
  return decode_common(out, q, k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       scale, dtype, partition_size, nullptr, workspace, workspace_bytes, false,
                       nullptr, 0, nullptr, 0, nullptr, true, stream, &sp);
}

int paged_attn_decode_store(void* out, const void* q, const void* key, int64_t key_token_stride,
                            const void* value, int64_t value_token_stride,
                            const int32_t* slot_mapping, void* k_cache, void* v_cache,
                            int32_t num_blocks, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, float scale, pkv_dtype_t dtype,
                            int32_t partition_size, const int32_t* kv_stream_from,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(out, q, k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       scale, dtype, partition_size, kv_stream_from, workspace, workspace_bytes,
                       true, key,
                       key_token_stride, value, value_token_stride, slot_mapping, true, stream);
}

int paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              int32_t num_blocks, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, float scale, pkv_dtype_t dtype,
                              int32_t partition_size, const int32_t* kv_stream_from,
                              hipStream_t stream) {
  // the bytes the call needs (0 when the arguments are invalid: decode_common reports why)
  const size_t need = num_seqs > 0 ? paged_attn_decode_workspace_bytes(
                                         num_seqs, num_heads, head_dim, max_blocks_per_seq,
                                         block_size, partition_size)
                                   : 0;
  if (need > (size_t)PKV_DECODE_NOALLOC_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_on_current_device(&ws);
    if (rc != PKV_OK) return rc;
  }
  return decode_common(out, q, k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       scale, dtype, partition_size, kv_stream_from, ws, need, false, nullptr, 0,
                       nullptr, 0, nullptr, false, stream);
}

// ------------------------------------------------------------------------- prefill
}  // extern "C"

namespace {

// The shared body of paged_attn_prefill_varlen and attn_prefill_varlen (packed: the latter;
// k / v then hold packed rows with the given token strides and no table is read).
int prefill_common(void* out, const void* q, const void* k, const void* v, int32_t num_blocks,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                   int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, float scale, int32_t causal, pkv_dtype_t dtype,
                   bool packed, int64_t k_stride, int64_t v_stride, hipStream_t stream) {
  if (dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (causal != 1) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0) return PKV_ERR_INVALID;
  if (!packed && (num_blocks < 0 || max_blocks_per_seq <= 0)) return PKV_ERR_INVALID;
  if (max_seqlen_k < max_seqlen_q) return PKV_ERR_INVALID;  // every Lk >= its Lq
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads) return PKV_ERR_INVALID;
  if (!packed && !pow2_at_least_16(block_size)) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (!supported_group(num_heads, num_kv_heads)) return PKV_ERR_UNSUPPORTED;
  if (!packed && (int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PKV_ERR_INVALID;
  // a 64-row tile is read with 32-bit byte offsets from its first row: 64 rows of at most
  // 2 * stride bytes each must stay below 2^31
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (row > (INT32_MAX >> 7)) return PKV_ERR_UNSUPPORTED;
  if (packed) {
    if (k_stride < row || v_stride < row || k_stride % 8 || v_stride % 8) return PKV_ERR_INVALID;
    if (k_stride > (INT32_MAX >> 7) || v_stride > (INT32_MAX >> 7)) return PKV_ERR_UNSUPPORTED;
  }
  // the launch has one plane per possible count of 64-key tiles of a unit
  const int64_t key_cap = packed ? INT32_MAX : (int64_t)max_blocks_per_seq * block_size;
  const int64_t key_tiles = ((max_seqlen_k < key_cap ? max_seqlen_k : key_cap) + 63) / 64;
  if (num_seqs > 65535 || key_tiles > 65535) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PKV_OK;
  if (!out || !q || !k || !v || !cu_seqlens_q || !cu_seqlens_k) return PKV_ERR_INVALID;
  if (!packed && !block_tables) return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v)) return PKV_ERR_INVALID;
  if (pkv::run_debug_checks(stream)) {
    const int chk = pkv_check_prefill(packed ? nullptr : block_tables, max_blocks_per_seq,
                                      cu_seqlens_q, cu_seqlens_k, num_seqs, total_q,
                                      max_seqlen_q, max_seqlen_k, num_blocks, block_size, 1,
                                      stream, nullptr);
    if (chk != PKV_OK) return chk;
  }
  pkv::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k;
  a.v_cache = v;
  a.num_blocks = packed ? 0 : num_blocks;
  a.block_tables = packed ? nullptr : block_tables;
  a.max_blocks_per_seq = packed ? 0 : max_blocks_per_seq;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.num_seqs = num_seqs;
  a.key_tiles = (int32_t)key_tiles;
  a.packed = packed ? 1 : 0;
  a.k_stride = k_stride;
  a.v_stride = v_stride;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = packed ? 0 : block_size;
  a.scale = scale;
  const int rc = pkv::launch_prefill(a, stream);
  return rc == 0 ? PKV_OK : (rc == -2 ? PKV_ERR_UNSUPPORTED : PKV_ERR_HIP);
}

}  // namespace

extern "C" {

int paged_attn_prefill_varlen(void* out, const void* q, const void* k_cache, const void* v_cache,
                              int32_t num_blocks, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              float scale, int32_t causal, pkv_dtype_t dtype,
                              hipStream_t stream) {
  return prefill_common(out, q, k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq,
                        cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, max_seqlen_q,
                        max_seqlen_k, num_heads, num_kv_heads, head_dim, block_size, scale,
                        causal, dtype, false, 0, 0, stream);
}

int attn_prefill_varlen(void* out, const void* q, const void* k, int64_t k_token_stride,
                        const void* v, int64_t v_token_stride, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q,
                        int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, float scale, int32_t causal,
                        pkv_dtype_t dtype, hipStream_t stream) {
  return prefill_common(out, q, k, v, 0, nullptr, 0, cu_seqlens_q, cu_seqlens_k, num_seqs,
                        total_q, max_seqlen_q, max_seqlen_k, num_heads, num_kv_heads, head_dim,
                        0, scale, causal, dtype, true, k_token_stride, v_token_stride, stream);
}

}  // extern "C"
