// Internal launchers behind the C ABI (argument validation happens in api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kDecodeDefaultPartition = 256;   // smallest share of keys per wavefront
constexpr int kDecodeMaxPartition = 1024;
constexpr int kDecodeDefaultWorkgroups = 512;  // 4 wavefronts each: 2 per SIMD on 256 CUs

int launch_store_kvcache(const void* key, int64_t key_stride, const void* value,
                         int64_t value_stride, void* k_cache, void* v_cache, int64_t num_slots,
                         const int32_t* slot_mapping, int32_t num_tokens, int32_t row_elems,
                         int32_t elem_bytes, hipStream_t stream);

// Decode partials of shared prefix blocks: group g is the sequences group_members[group_ptr[g]
// .. group_ptr[g+1]-1], each holding the same block in table column group_col[g].
struct PrefixArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  int32_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* group_ptr;
  const int32_t* group_members;
  const int32_t* group_col;
  int32_t num_groups, max_group_size;
  int32_t num_heads, num_kv_heads, head_dim, block_size;
  float scale;
  float* pfx_o;   // [num_seqs, Hq, max_blocks_per_seq, D]: slot (b, h, column)
  float* pfx_ml;  // [num_seqs, Hq, max_blocks_per_seq, 2]
};
int launch_decode_prefix(const PrefixArgs& a, hipStream_t stream);

// What the combine kernel reads of the shared blocks' pieces (cols == nullptr: none).
struct PrefixParts {
  const int32_t* cols;  // [num_seqs]: shared leading table columns of each sequence
  const float* o;       // PrefixArgs::pfx_o
  const float* ml;      // PrefixArgs::pfx_ml
  int32_t stride;       // slots per (sequence, head): max_blocks_per_seq
  int32_t bs_log2;
};

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  int32_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  int32_t num_seqs, num_heads, num_kv_heads, head_dim, block_size;
  float scale;
  int32_t bf16;             // 1 = bf16, 0 = fp32
  int32_t partition;        // smallest share of keys per wavefront (min_keys)
  int32_t max_parts;        // partial slots per (sequence, head): ceil(cap / partition) + 1
  float* ws_o;              // [num_seqs, Hq, max_parts, D]
  float* ws_ml;             // [num_seqs, Hq, max_parts, 2]
  int32_t* ws_meta;         // [num_seqs + 2]: the share size, then the context prefix sums
  int32_t max_workgroups;   // cap of the decode grid (4 wavefronts each)
  const int32_t* kv_stream_from;  // [num_seqs] or null: columns >= [b] read non-temporally
  // fused store of the step's tokens (new_k == nullptr: attention only); token b of
  // new_k / new_v is the newest token of sequence b, written to slot slot_mapping[b]
  const void* new_k;
  int64_t new_k_stride;     // elements between tokens
  const void* new_v;
  int64_t new_v_stride;
  const int32_t* slot_mapping;
  int64_t num_slots;
  // prefix mode: kv_stream_from[b] is sequence b's count of shared leading table columns,
  // whose keys the decode_prefix_unit work units take (pfx); the stream kernel takes the rest
  int32_t prefix;
  PrefixArgs pfx;
};

// What the combine kernel needs for the fused store (key == nullptr: not fused).
struct NewTokens {
  const void* q;
  const void* key;
  int64_t key_stride;
  const void* value;
  int64_t value_stride;
  const int32_t* slot_mapping;
  void* k_cache;
  void* v_cache;
  int64_t num_slots;
  float scale_log2e;
};
int launch_decode(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  int32_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t num_seqs;
  int32_t key_tiles;         // grid planes: ceil(min(max_seqlen_k, table capacity) / 64)
  int32_t packed;            // 1: k_cache / v_cache are packed K / V rows, no block table
  int64_t k_stride, v_stride;  // packed: token strides in elements
  int32_t num_heads, num_kv_heads, head_dim, block_size;
  float scale;
};
int launch_prefill(const PrefillArgs& a, hipStream_t stream);


}  // namespace pkv
