/*
 * paged_kv.h - C ABI of the paged-attention hot path for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the nano-vLLM engine described on three pages:
 *   [P1] "vLLM 学习笔记 02：nano-vllm 源码逐段精读" (listings ModelRunner.prepare_prefill,
 *        prepare_block_tables, prepare_decode, store_kvcache, Attention.forward, Context)
 *   [P2] "Nano-vLLM代码手撕笔记" (sections 请求执行 – 输入序列预处理与context构建,
 *        请求执行 – run model, cuda graph捕捉与context设置)
 *   [P3] "Nano-vLLM 代码解析" (section 4.2.1 输入准备)
 *
 * Conventions for every call:
 *   - Sizes are element counts unless named *_bytes. Hq = num_heads, Hkv = num_kv_heads,
 *     D = head_dim, bs = block_size, G = Hq / Hkv.
 *   - The paged cache of one layer is a pair of arrays k_cache, v_cache of shape
 *     [num_blocks, bs, Hkv, D], contiguous: physical slot s = block * bs + offset holds
 *     Hkv * D contiguous elements ([P1] store_kvcache asserts; [P1] allocate_kv_cache).
 *   - Query head h reads kv head h / G (contiguous head groups, as tensor parallelism
 *     splits heads in [P1] QKVParallelLinear).
 *   - "device" pointers are HIP device memory owned by the caller; the library never
 *     allocates, frees or keeps them. "host" pointers are ordinary host memory.
 *   - Device calls enqueue on `stream` (0 = the null stream) and never synchronise the host.
 *   - Every call returns PKV_OK or a negative status; nothing throws across the ABI.
 *     Host-checkable argument errors are reported before anything is enqueued.
 *     Data-dependent preconditions (slot and block-id ranges, lengths) are documented
 *     per call; the kernels bounds-check them so that a violation never reads or writes
 *     outside the caller's arrays (see each call for what it does instead). pkv_check_*
 *     (near the end of this file) test them on request and name the first violation.
 */
#ifndef PAGED_KV_H_
#define PAGED_KV_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the tensors of a call. The two range entries are not types: they make
 * every int32 value a valid pkv_dtype_t (and fix its size at 32 bits), so that a value the
 * library does not support is reported as PKV_ERR_UNSUPPORTED instead of being undefined. */
typedef enum {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_DTYPE_RANGE_MIN_ = INT32_MIN,
  PKV_DTYPE_RANGE_MAX_ = INT32_MAX
} pkv_dtype_t;

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,     /* null pointer, negative size, inconsistent arguments */
  PKV_ERR_UNSUPPORTED = -2, /* a valid shape or dtype the library does not implement */
  PKV_ERR_WORKSPACE = -3,   /* decode workspace smaller than the query function asks */
  PKV_ERR_HIP = -4,         /* a HIP launch error */
  PKV_ERR_PRECONDITION = -5 /* a data-dependent precondition does not hold (pkv_check_*, or
                               a device call made with PKV_DEBUG set) */
};

/* Human-readable name of a status code (static storage). */
const char* pkv_status_string(int status);

/* ------------------------------------------------------------------------------------
 * Host metadata (the harness step before the kernels).
 *
 * pkv_prefill_metadata - [P1] ModelRunner.prepare_prefill and prepare_block_tables;
 * pinned by the worked example of [P2] 请求执行 – 输入序列预处理与context构建.
 * Sequence b computes positions start = num_cached[b] .. end-1, end = start + num_scheduled[b]
 * (start may fall inside a block). Outputs, all host memory:
 *   cu_seqlens_q[num_seqs+1], cu_seqlens_k[num_seqs+1]: prefix sums of end-start and end;
 *   *max_seqlen_q, *max_seqlen_k;
 *   slot_mapping[total_q], positions[total_q] (int64): for each computed position p of
 *     each sequence in order, slot = table[p / bs] * bs + p % bs and p itself;
 *   block_tables[num_seqs * table_width]: each table copied and padded with -1.
 * Inputs: block tables are ragged, sequence b's ids are
 *   block_table_flat[block_table_offsets[b] .. block_table_offsets[b+1]-1].
 * slot_capacity may be 0 to skip the check of slot_mapping's size (the caller vouches that it
 * holds total_q entries); positions may be NULL to skip that output.
 * Errors: PKV_ERR_INVALID if a table holds fewer than ceil(end / bs) ids, if a table is
 * longer than table_width, if total_q exceeds slot_capacity, or on negative counts.
 * -------------------------------------------------------------------------------------*/
int pkv_prefill_metadata(int32_t num_seqs, const int32_t* num_cached, const int32_t* num_scheduled,
                         const int32_t* block_table_flat, const int64_t* block_table_offsets,
                         int32_t block_size, int32_t table_width,
                         int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                         int32_t* max_seqlen_q, int32_t* max_seqlen_k,
                         int32_t* slot_mapping, int64_t slot_capacity, int64_t* positions,
                         int32_t* block_tables);

/* pkv_decode_metadata - [P1] ModelRunner.prepare_decode, Sequence.last_block_num_tokens;
 * pinned by [P2]'s decode continuation of the same worked example.
 * Sequence b has seq_lens[b] = len(seq) >= 1 tokens, the newest one being computed:
 *   slot_mapping[b] = last table entry * bs + last_block_num_tokens - 1,
 *   context_lens[b] = seq_lens[b], positions[b] = seq_lens[b] - 1 (int64, may be NULL),
 *   block_tables[num_seqs * table_width] padded with -1.
 * Errors: PKV_ERR_INVALID unless every table holds exactly ceil(len / bs) ids (so its last
 * entry is the newest token's block) and fits table_width. All pointers are host memory. */
int pkv_decode_metadata(int32_t num_seqs, const int32_t* seq_lens,
                        const int32_t* block_table_flat, const int64_t* block_table_offsets,
                        int32_t block_size, int32_t table_width,
                        int32_t* slot_mapping, int32_t* context_lens, int64_t* positions,
                        int32_t* block_tables);

/* ------------------------------------------------------------------------------------
 * store_kvcache - [P1] store_kvcache / store_kvcache_kernel; [P2] 请求执行 – run model.
 * For every token t < num_tokens with s = slot_mapping[t] != -1, copies the Hkv*D elements
 * of key row t into k_cache slot s and those of value row t into v_cache slot s, bit for bit.
 *   key, value   device, [num_tokens, Hkv, D] with token stride *_token_stride elements,
 *                head stride D and unit element stride (a view into a fused qkv buffer works).
 *   k_cache, v_cache  device, [num_slots, Hkv * D] (= [num_blocks, bs, Hkv, D] flattened).
 *   slot_mapping device int32 [num_tokens]; -1 = skip (padding or a prefix-cache hit).
 *   dtype        PKV_F32 or PKV_BF16 (key, value and the caches share it).
 * Preconditions: non-negative slots are unique within the call (the engine hands each
 * token its own slot); a slot >= num_slots or < -1 is skipped and nothing is written for it.
 * num_tokens == 0 is a no-op. Any token stride works; 16-byte aligned rows take the
 * vector path. Errors: PKV_ERR_INVALID (null pointers, negative sizes, token stride
 * smaller than Hkv*D), PKV_ERR_UNSUPPORTED (dtype), PKV_ERR_HIP.
 * -------------------------------------------------------------------------------------*/
int store_kvcache(const void* key, int64_t key_token_stride,
                  const void* value, int64_t value_token_stride,
                  void* k_cache, void* v_cache, int64_t num_slots,
                  const int32_t* slot_mapping, int32_t num_tokens,
                  int32_t num_kv_heads, int32_t head_dim, pkv_dtype_t dtype,
                  hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Decode attention - [P1] Attention.forward (decode branch, flash_attn_with_kvcache with
 * cache_seqlens = context_lens and a block table); [P1] prepare_decode for the meaning of
 * context_lens (len(seq), the newest token included: its K/V is stored before attention).
 *
 * For sequence b with n = context_lens[b] and every q head h (kv head g = h / G):
 *   out[b,h,:] = sum_{j<n} softmax_j(scale * <q[b,h,:], K_b[j,g,:]>) V_b[j,g,:]
 * where K_b[j] is k_cache[block_tables[b * max_blocks_per_seq + j / bs], j % bs].
 * The (sequence, kv head) key segments are laid end to end and every wavefront takes an equal
 * contiguous share of them (never fewer than `partition_size` keys); a segment cut between
 * shares is merged exactly afterwards from per-share (max, sum, weighted V) partials (split-K
 * softmax), so the result does not depend on how the keys were split beyond rounding.
 *   out          device [num_seqs, Hq, D], dtype
 *   q            device [num_seqs, Hq, D], dtype, contiguous
 *   k_cache, v_cache  device [num_blocks, bs, Hkv, D], dtype
 *   block_tables device int32 [num_seqs, max_blocks_per_seq]; entries at or past
 *                ceil(n / bs) are never read (padding -1 or stale ids are fine).
 *   context_lens device int32 [num_seqs]; 0 gives a zero output row without reading memory.
 *   partition_size  smallest share of keys per wavefront, a multiple of 64 in [64, 1024];
 *                0 = library default: 64 keys when num_seqs * max_blocks_per_seq * bs
 *                < 65536, 128 up to 131072, 256 above (a small batch then spreads over
 *                more workgroups). It also sizes the workspace.
 *   workspace    device scratch of at least paged_attn_decode_workspace_bytes(...) bytes
 *                (same num_seqs, heads, head_dim, max_blocks_per_seq, block_size and
 *                partition_size; with partition_size 0 the bytes for num_seqs also cover
 *                every call with fewer sequences), owned by the caller; no initial
 *                contents needed; in use until the stream passes the end of the call, so
 *                calls that overlap on different streams need different workspaces.
 *   kv_stream_from  NULL or device int32 [num_seqs]: per sequence, the first block-table
 *                column whose K/V rows are read with non-temporal loads (see below); it
 *                changes no result.
 * out, q, k_cache, v_cache and workspace must be 16-byte aligned (PKV_ERR_INVALID otherwise).
 * Preconditions: num_blocks >= 1; n <= max_blocks_per_seq * bs (larger n is clamped to
 * that); table entries below ceil(n / bs) lie in [0, num_blocks) - an entry outside it is
 * not dereferenced and turns that sequence's output row into NaN.
 * Supported: dtype PKV_F32 or PKV_BF16; D in {64, 128}; G in {1, 2, 4, 8}; bs a power of
 * two >= 16; num_seqs <= 16383 and num_seqs * max_blocks_per_seq * bs * Hkv < 2^31.
 * Errors: PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP.
 * -------------------------------------------------------------------------------------*/
size_t paged_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                         int32_t max_blocks_per_seq, int32_t block_size,
                                         int32_t partition_size);

/* kv_stream_from - how a decode call (paged_attn_decode, paged_attn_decode_store,
 * paged_attn_decode_noalloc and the steps recorded by pkv_decode_graphs_create) reads the
 * cached K/V rows; an argument of each call, so calls on different threads or streams never
 * affect each other. NULL: every row with ordinary loads. Otherwise a device int32 array
 * [num_seqs]: sequence b's rows of block-table columns >= kv_stream_from[b] are read with
 * non-temporal loads (they stream past the caches without displacing other lines), the
 * others with ordinary loads. A tuning choice for the caller, who knows from its block
 * manager's reference counts which leading blocks of each table other sequences of the batch
 * also read (prefix caching shares only leading full blocks): pass each sequence's count of
 * shared leading blocks - 0 when no block of the batch is read twice - so that the shared
 * blocks stay cached for their other readers while the private rows stream. Measured on the
 * batch-64 workload (non-overlapping tables, all 0, 4 layer pools rotated): 109.6 -> 98.1 us
 * per call. Any value (negative: all streamed; >= the table width: none) is valid, and the
 * outputs are bitwise the same for every choice. The array is read at run time, like
 * context_lens, so a recorded graph follows its contents. */

int paged_attn_decode(void* out, const void* q,
                      const void* k_cache, const void* v_cache, int32_t num_blocks,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, float scale, pkv_dtype_t dtype,
                      int32_t partition_size, const int32_t* kv_stream_from,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * paged_attn_decode_noalloc - for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * operation and arguments as paged_attn_decode, without the workspace. The call allocates
 * nothing; its split-K partials go to a library-owned device array of
 * PKV_DECODE_NOALLOC_SCRATCH_BYTES, one per GPU, held from the library's first use on that
 * GPU until the process ends (its address is looked up on the first call on each device).
 * Results are bitwise those of paged_attn_decode with the same arguments.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents (no
 * call needs it to start in any particular state): calls that overlap on one GPU - on
 * different streams, or from different threads without ordering between their streams -
 * race and may give wrong outputs. Calls on different GPUs never share it.
 * Errors: as paged_attn_decode; PKV_ERR_WORKSPACE when the call would need more than
 * PKV_DECODE_NOALLOC_SCRATCH_BYTES (paged_attn_decode_workspace_bytes with the same
 * arguments reports the need; e.g. 9.1 MB for 64 sequences, 16 q heads, D 128 and
 * 16 blocks of 256 keys per table); PKV_ERR_HIP if the array's address cannot be found.
 * -------------------------------------------------------------------------------------*/
#define PKV_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)
int paged_attn_decode_noalloc(void* out, const void* q,
                              const void* k_cache, const void* v_cache, int32_t num_blocks,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, float scale, pkv_dtype_t dtype,
                              int32_t partition_size, const int32_t* kv_stream_from,
                              hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Decode attention with shared prefix blocks read once - [P1] Attention.forward, decode
 * branch, for a batch whose block tables share leading blocks ([P1] BlockManager.allocate:
 * a cached block is reused by every sequence whose token prefix hashes to it, so only
 * leading full blocks are shared, each in the same table column of all its sharers).
 * Same operation and arguments as paged_attn_decode (attention only), except that:
 *   shared_cols  device int32 [num_seqs]: sequence b's count of shared leading columns
 *                (0 = none); its keys from shared_cols[b] * bs on go through the split-K
 *                stream (read with non-temporal loads), the keys before through the groups.
 *   group_ptr, group_members, group_col  device int32 arrays describing the groups: group
 *                g is sequences group_members[group_ptr[g] .. group_ptr[g+1]-1], all holding
 *                one block in table column group_col[g]; [num_groups + 1], [group_ptr[
 *                num_groups]] and [num_groups] entries. Each group's block is read once per
 *                64 members and its keys multiplied out with bf16 MFMA for all of them.
 *   num_groups, max_group_size  host ints: the group count and an upper bound of every
 *                group's member count (it sizes the launch).
 *   workspace    at least paged_attn_decode_prefix_workspace_bytes(...) bytes (the decode
 *                call's slots plus (D + 2) floats per (sequence, q head, table column)).
 * Preconditions: the (member, group column) pairs of the groups are exactly the pairs
 * (b, c) with c < shared_cols[b], each once; every member of a group holds the same block
 * id in that column; shared_cols[b] * bs <= context_lens[b] - 1 (the newest token's block
 * is private). A column left without a group is merged from whatever its slot holds; a
 * member, group column or shared_cols value out of range makes the kernels read and write
 * outside their arrays. pkv_check_prefix (and PKV_DEBUG) names such mistakes.
 * Supported: bf16 only; block_size >= 64; Hkv * D < 2^24; num_groups <= 65535; the decode
 * call's other limits. Results equal paged_attn_decode's within rounding: the shared keys'
 * probabilities are rounded to bf16 for the MFMA, as in prefill. Errors as
 * paged_attn_decode.
 * -------------------------------------------------------------------------------------*/
size_t paged_attn_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                                int32_t head_dim, int32_t max_blocks_per_seq,
                                                int32_t block_size, int32_t partition_size);
int paged_attn_decode_prefix(void* out, const void* q,
                             const void* k_cache, const void* v_cache, int32_t num_blocks,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, float scale, pkv_dtype_t dtype,
                             int32_t partition_size, const int32_t* shared_cols,
                             const int32_t* group_ptr, const int32_t* group_members,
                             const int32_t* group_col, int32_t num_groups,
                             int32_t max_group_size, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Decode attention with the step's store fused in - [P1] Attention.forward, decode branch:
 * store_kvcache of the step's K/V rows, then the decode attention over the cache.
 * Same result as store_kvcache(key, value, k_cache, v_cache, slot_mapping[0 .. num_seqs))
 * followed by paged_attn_decode(...) with the same arguments, up to rounding: token b of
 * key / value is the newest token of sequence b (position context_lens[b] - 1), so the
 * attention takes that token's K/V from key / value and the other context_lens[b] - 1
 * keys from the cache, and the rows are written to slot slot_mapping[b] of the caches
 * (bit for bit; -1 or a slot >= num_blocks * block_size is skipped) within the call.
 *   key, value   device [num_seqs, Hkv, D], dtype, token stride *_token_stride elements
 *                (>= Hkv * D; stride * element size a multiple of 16 bytes), 16-byte aligned.
 *   slot_mapping device int32 [num_seqs] ([P1] prepare_decode's slot of the newest token).
 *   Other arguments, the workspace and its size: as paged_attn_decode.
 * Preconditions: those of paged_attn_decode and store_kvcache; slot_mapping[b] is the slot
 * of position context_lens[b] - 1 in sequence b's block table (then the cache ends up as
 * after the two separate calls). Sequences with context_lens[b] == 0 get a zero row; their
 * rows are still stored if their slot is valid.
 * Errors: as paged_attn_decode, plus PKV_ERR_INVALID for null key / value / slot_mapping
 * or a stride or alignment outside the rules above.
 * -------------------------------------------------------------------------------------*/
int paged_attn_decode_store(void* out, const void* q,
                            const void* key, int64_t key_token_stride,
                            const void* value, int64_t value_token_stride,
                            const int32_t* slot_mapping,
                            void* k_cache, void* v_cache, int32_t num_blocks,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, float scale, pkv_dtype_t dtype,
                            int32_t partition_size, const int32_t* kv_stream_from,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Decode steps replayed from captured HIP graphs - [P1] ModelRunner.capture_cudagraph and
 * run_model; [P2] cuda graph捕捉与context设置 (why: a recorded graph fixes shapes and device
 * addresses, and one graph launch replaces the step's kernel launches).
 *
 * pkv_decode_graphs_create records one paged_attn_decode_store call per batch bucket
 * (1, 2, 4, 8, then every multiple of 16 up to max_batch, plus max_batch itself when it is
 * not a multiple of 16) over caller-owned static buffers sized for max_batch rows:
 *   out, q       device [max_batch, Hq, D]; key, value device [max_batch, Hkv, D] with
 *                token strides; slot_mapping, context_lens device int32 [max_batch];
 *   block_tables device int32 [max_batch, max_blocks_per_seq];
 *   workspace    device, >= paged_attn_decode_workspace_bytes(max_batch, ...) bytes.
 * The other arguments are those of paged_attn_decode_store. Recording launches nothing.
 * pkv_decode_graphs_launch(h, B, stream) replays, on `stream`, the graph of the smallest
 * bucket >= B: it computes rows 0 .. bucket-1 of the buffers as they hold at that point in
 * the stream. As in [P1] run_model, the caller writes the step's B rows and pads rows
 * B .. bucket-1 with context_lens 0 and slot_mapping -1 (they get zero rows and store
 * nothing; their block-table rows are never read). Every data-dependent quantity is
 * computed on the device at run time, so any lengths up to max_blocks_per_seq * bs work.
 * Ownership: the handle owns the graphs only; the buffers stay the caller's and must
 * outlive the handle. One replay at a time per handle (replays share the workspace).
 * pkv_decode_graphs_bucket(h, B) returns that bucket (or a negative status);
 * pkv_decode_graphs_count / _buckets report the bucket list (ascending).
 * Errors: PKV_ERR_INVALID (null handle, max_batch outside 1 .. 16383, B outside
 * 1 .. max_batch), PKV_ERR_WORKSPACE, any status paged_attn_decode_store returns for the
 * recorded call, PKV_ERR_HIP (capture, instantiation or launch failed). On error, create
 * leaves *handle NULL and frees what it made.
 *
 * pkv_decode_graphs_create_layers records a whole decode step of a model with num_layers
 * attention layers, the unit [P1] capture_cudagraph records: each bucket's graph holds
 * num_layers paged_attn_decode_store calls in layer order on one stream. Every layer has
 * its own pool and its own rows: out[l], q[l], key[l], value[l], k_cache[l], v_cache[l] are
 * host arrays of num_layers device pointers (read during the call only; the buffers they
 * name are as above, one set per layer). slot_mapping, block_tables, context_lens and
 * kv_stream_from are shared by all layers, as every layer of [P1]'s model reads the one
 * step Context (one block id names the same block in every layer's pool). The layers run
 * one after another and share the workspace. pkv_decode_graphs_create is this call with
 * num_layers 1. Errors as above, plus PKV_ERR_INVALID for num_layers outside 1 .. 1024 or
 * a null pointer array.
 * -------------------------------------------------------------------------------------*/
typedef struct pkv_decode_graphs pkv_decode_graphs;

int pkv_decode_graphs_create(pkv_decode_graphs** handle, int32_t max_batch,
                             void* out, const void* q,
                             const void* key, int64_t key_token_stride,
                             const void* value, int64_t value_token_stride,
                             const int32_t* slot_mapping,
                             void* k_cache, void* v_cache, int32_t num_blocks,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, float scale, pkv_dtype_t dtype,
                             int32_t partition_size, const int32_t* kv_stream_from,
                             void* workspace, size_t workspace_bytes);
int pkv_decode_graphs_create_layers(pkv_decode_graphs** handle, int32_t max_batch,
                                    int32_t num_layers,
                                    void* const* out, const void* const* q,
                                    const void* const* key, int64_t key_token_stride,
                                    const void* const* value, int64_t value_token_stride,
                                    const int32_t* slot_mapping,
                                    void* const* k_cache, void* const* v_cache,
                                    int32_t num_blocks,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens,
                                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, float scale, pkv_dtype_t dtype,
                                    int32_t partition_size, const int32_t* kv_stream_from,
                                    void* workspace, size_t workspace_bytes);
int pkv_decode_graphs_count(const pkv_decode_graphs* handle);
int pkv_decode_graphs_buckets(const pkv_decode_graphs* handle, int32_t* buckets,
                              int32_t capacity);
int pkv_decode_graphs_bucket(const pkv_decode_graphs* handle, int32_t batch);
int pkv_decode_graphs_launch(pkv_decode_graphs* handle, int32_t batch, hipStream_t stream);
int pkv_decode_graphs_destroy(pkv_decode_graphs* handle);

/* ------------------------------------------------------------------------------------
 * Varlen causal prefill - [P1] Attention.forward (prefill branch, flash_attn_varlen_func
 * with block_table, causal=True); [P1] prepare_prefill for cu_seqlens; [P2] 请求执行 –
 * 输入序列预处理与context构建 for prefix-cache hits (keys cover more tokens than queries).
 *
 * Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (Lq of them) and
 * Lk = cu_seqlens_k[b+1] - cu_seqlens_k[b] keys read through its block table, Lk >= Lq.
 * Query i of the sequence sits at position Lk - Lq + i and attends keys 0 .. Lk - Lq + i
 * (causal, aligned at the bottom right, so cached prefix tokens are visible to all).
 *   out, q       device [total_q, Hq, D] bf16, contiguous (packed sequences)
 *   k_cache, v_cache  device [num_blocks, bs, Hkv, D] bf16 (the new tokens already stored)
 *   block_tables device int32 [num_seqs, max_blocks_per_seq]
 *   cu_seqlens_q, cu_seqlens_k  device int32 [num_seqs + 1]
 *   max_seqlen_q, max_seqlen_k  host ints: upper bounds of every Lq and every Lk (the
 *                engine's Context carries both); max_seqlen_k sizes the launch, which has
 *                one plane of workgroups per possible count of 64-key tiles.
 *   causal       must be 1 (the engine always attends causally).
 * out, q, k_cache and v_cache must be 16-byte aligned (PKV_ERR_INVALID otherwise).
 * Preconditions: cu_seqlens_q[num_seqs] == total_q; Lq <= max_seqlen_q; Lk >= Lq;
 * Lk <= max_seqlen_k (a sequence breaking this may have rows left unwritten);
 * Lk <= max_blocks_per_seq * bs (larger Lk is clamped); table entries below
 * ceil(Lk / bs) lie in [0, num_blocks) - an entry outside it is not
 * dereferenced; it turns into NaN every output row of that sequence that attends a key in
 * that block, and may do the same to other rows of that sequence sharing a 64-row query
 * tile with one (tiles are counted back from the sequence's last row). Rows of other
 * sequences are unaffected.
 * Supported: bf16 only (fp32 accumulation); D in {64, 128}; G in {1, 2, 4, 8}; bs a power
 * of two >= 16; Hkv * D < 2^24; num_seqs <= 65535 and
 * ceil(min(max_seqlen_k, max_blocks_per_seq * bs) / 64) <= 65535. Errors: PKV_ERR_INVALID (also max_seqlen_k < max_seqlen_q),
 * PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.
 * -------------------------------------------------------------------------------------*/
int paged_attn_prefill_varlen(void* out, const void* q,
                              const void* k_cache, const void* v_cache, int32_t num_blocks,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t num_seqs, int32_t total_q,
                              int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, float scale, int32_t causal,
                              pkv_dtype_t dtype, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Varlen causal prefill over packed K/V - [P1] Attention.forward, prefill branch when the
 * context holds no block tables (no prefix-cache hit): flash_attn_varlen_func on the step's
 * own k and v instead of the caches.
 * Same operation as paged_attn_prefill_varlen, except that sequence b's keys are rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v (Lk of them) rather than positions read
 * through a block table.
 *   out, q       device [total_q, Hq, D] bf16, contiguous (packed sequences)
 *   k, v         device [rows, Hkv, D] bf16 with token strides *_token_stride elements
 *                (>= Hkv * D, multiples of 8, so every row starts on 16 bytes; head stride D,
 *                unit element stride - a view into a fused qkv buffer works)
 *   cu_seqlens_q, cu_seqlens_k  device int32 [num_seqs + 1]
 *   max_seqlen_q, max_seqlen_k  host ints: upper bounds of every Lq and every Lk; max_seqlen_k
 *                sizes the launch (one plane of workgroups per possible count of 64-key tiles)
 *   causal       must be 1.
 * out, q, k and v must be 16-byte aligned (PKV_ERR_INVALID otherwise).
 * Preconditions: cu_seqlens_q[num_seqs] == total_q; Lq <= max_seqlen_q; Lk >= Lq;
 * Lk <= max_seqlen_k (a sequence breaking this may have rows left unwritten); the rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 exist in k and v.
 * Supported: bf16 only (fp32 accumulation); D in {64, 128}; G in {1, 2, 4, 8};
 * num_seqs <= 65535; ceil(max_seqlen_k / 64) <= 65535; token strides < 2^24 elements.
 * Errors: PKV_ERR_INVALID (also max_seqlen_k < max_seqlen_q, bad strides or alignment),
 * PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.
 * -------------------------------------------------------------------------------------*/
int attn_prefill_varlen(void* out, const void* q,
                        const void* k, int64_t k_token_stride,
                        const void* v, int64_t v_token_stride,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t num_seqs, int32_t total_q,
                        int32_t max_seqlen_q, int32_t max_seqlen_k,
                        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        float scale, int32_t causal, pkv_dtype_t dtype,
                        hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Checks of the data-dependent preconditions - [P1] store_kvcache (its wrapper asserts the
 * shapes before the scatter; the engine's block manager and prepare_* build the rest of the
 * metadata, which the kernels trust).
 *
 * Each check reads the metadata a call would use and returns PKV_OK, or
 * PKV_ERR_PRECONDITION with *first (if not NULL) naming the first violation found; it
 * computes nothing else. With on_device 0 the arrays are host memory; with on_device 1
 * they are device memory, copied to the host on `stream` first, which synchronises the
 * stream (PKV_ERR_INVALID while the stream records a graph, PKV_ERR_HIP if the copy fails).
 * *first is zeroed on entry.
 *   pkv_check_store     store_kvcache's slot_mapping [num_tokens] against num_slots:
 *                       every slot is -1 or in [0, num_slots) (SLOT_RANGE, index = token);
 *                       non-negative slots are unique (SLOT_DUPLICATE, index = the earliest
 *                       token whose slot an earlier token already has).
 *   pkv_check_decode    a decode call's context_lens [num_seqs] and block_tables: every
 *                       length in [0, max_blocks_per_seq * bs] (CONTEXT_RANGE, index = b);
 *                       the first ceil(n_b / bs) entries of each table in [0, num_blocks)
 *                       (BLOCK_RANGE, index = b * max_blocks_per_seq + column). With
 *                       slot_mapping (paged_attn_decode_store's, [num_seqs]; else NULL):
 *                       its slots as for a store, and each slot is -1 or the slot of the
 *                       sequence's newest position n_b - 1 under its own table, never set
 *                       for n_b = 0 (NEW_TOKEN_SLOT, index = b).
 *   pkv_check_prefill   a prefill call's cu_seqlens_q/k [num_seqs + 1]: cu_seqlens_q starts
 *                       at 0, both never decrease and cu_seqlens_q[num_seqs] == total_q
 *                       (CU_SEQLENS, index = the entry); Lk >= Lq (LK_LT_LQ, index = b);
 *                       Lq <= max_seqlen_q and Lk <= max_seqlen_k (MAX_SEQLEN); with
 *                       block_tables (NULL for attn_prefill_varlen's packed keys) also
 *                       Lk <= max_blocks_per_seq * bs (CONTEXT_RANGE) and the first
 *                       ceil(Lk / bs) entries of each table in [0, num_blocks) (BLOCK_RANGE).
 *   pkv_check_prefix    paged_attn_decode_prefix's groups, with the call's block_tables
 *                       and context_lens: each shared_cols[b] in [0, max_blocks_per_seq] and,
 *                       when above 0, shared_cols[b] * bs <= n_b - 1 (SHARED_COLS, index =
 *                       b); group_ptr starts at 0, never decreases, no group holds more than
 *                       max_group_size members and group_ptr[num_groups] is the number of
 *                       shared pairs, the sum of shared_cols (GROUP_PTR, index = the entry);
 *                       group_col[g] in [0, max_blocks_per_seq) (GROUP_COL, index = g); every
 *                       member in [0, num_seqs) (GROUP_MEMBER, index = its entry in
 *                       group_members); the (member, group_col[g]) pairs are exactly the
 *                       pairs (b, c) with c < shared_cols[b], each once (PREFIX_COVER, index
 *                       = b, value = c, at the entry that repeats a pair or names a column
 *                       outside b's shared ones); the members of a group hold one block id
 *                       in its column (GROUP_BLOCK, index = the entry, value = its id).
 * PKV_DEBUG: when this environment variable is set to a non-empty value other than "0" at
 * the library's first device call, store_kvcache, paged_attn_decode,
 * paged_attn_decode_store, paged_attn_decode_prefix (the decode check, then the prefix
 * check), paged_attn_prefill_varlen and attn_prefill_varlen run the
 * matching check on their device arrays (on_device 1) after their argument checks and
 * return its status without enqueuing anything when it fails. Such calls synchronise their
 * stream; while the stream records a graph the check is skipped. paged_attn_decode_noalloc
 * never checks (its callers cannot afford the copy).
 * -------------------------------------------------------------------------------------*/
enum {
  PKV_CHECK_SLOT_RANGE = 1,
  PKV_CHECK_SLOT_DUPLICATE = 2,
  PKV_CHECK_CONTEXT_RANGE = 3,
  PKV_CHECK_BLOCK_RANGE = 4,
  PKV_CHECK_NEW_TOKEN_SLOT = 5,
  PKV_CHECK_CU_SEQLENS = 6,
  PKV_CHECK_LK_LT_LQ = 7,
  PKV_CHECK_MAX_SEQLEN = 8,
  PKV_CHECK_SHARED_COLS = 9,
  PKV_CHECK_GROUP_PTR = 10,
  PKV_CHECK_GROUP_COL = 11,
  PKV_CHECK_GROUP_MEMBER = 12,
  PKV_CHECK_PREFIX_COVER = 13,
  PKV_CHECK_GROUP_BLOCK = 14
};

typedef struct pkv_violation {
  int32_t check;     /* PKV_CHECK_* (0: none) */
  int32_t reserved;  /* 0 */
  int64_t index;     /* where: token, sequence, table entry or cu_seqlens entry */
  int64_t value;     /* the offending value */
} pkv_violation;

int pkv_check_store(const int32_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                    int32_t on_device, hipStream_t stream, pkv_violation* first);
int pkv_check_decode(const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* slot_mapping, int32_t num_seqs,
                     int32_t num_blocks, int32_t block_size, int32_t on_device,
                     hipStream_t stream, pkv_violation* first);
int pkv_check_prefill(const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                      int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                      int32_t max_seqlen_k, int32_t num_blocks, int32_t block_size,
                      int32_t on_device, hipStream_t stream, pkv_violation* first);
int pkv_check_prefix(const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                     const int32_t* shared_cols, const int32_t* group_ptr,
                     const int32_t* group_members, const int32_t* group_col, int32_t num_groups,
                     int32_t max_group_size, int32_t on_device, hipStream_t stream,
                     pkv_violation* first);

/* ------------------------------------------------------------------------------------
 * Temperature sampling - [P3] section 4.3 采样器 (Sampler.forward); [P1] SamplingParams
 * (temperature > 1e-10) and ModelRunner.prepare_sample / run (one temperature per row).
 * For each row r: tokens[r] = argmax_i softmax(logits[r] / T_r)_i / max(E_ri, 1e-10) with
 * E_ri ~ Exp(1) independent, i.e. a draw from softmax(logits[r] / T_r). Computed as the
 * first index of the largest s_i = logits[r, i] / T_r - log(max(E_ri, 1e-10)) (the softmax
 * denominator does not change the winner).
 * E_ri = -log(u), u = (b + 0.5) / 2^23, b = the top 23 bits of a 32-bit word of
 * Philox4x64-10 (Salmon et al., SC 2011) with key (seed, 0) and counter (i / 8, r, offset,
 * 0): word (i % 8) / 2 of the block, low half for even i, high half for odd i. The caller
 * advances `offset` (e.g. once per step) for fresh draws with one seed.
 *   tokens       device int32 [num_rows] (output)
 *   logits       device [num_rows, row_stride] (first vocab_size columns used), fp32 or bf16;
 *                rows starting on 16 bytes are read with vector loads, others element-wise
 *   temperatures device fp32 [num_rows], each > 0
 *   workspace    device, >= pkv_sample_workspace_bytes(num_rows, vocab_size), 16-byte aligned
 * Scores are fp32 (the kernel's precision): among candidates whose scores differ by less
 * than fp32 rounding, either may be returned. NaN logits never win; a row with no finite
 * score returns 0. num_rows == 0 is a no-op.
 * Errors: PKV_ERR_INVALID (null pointers, row_stride < vocab_size),
 * PKV_ERR_UNSUPPORTED (dtype, num_rows > 65535), PKV_ERR_WORKSPACE, PKV_ERR_HIP.
 * -------------------------------------------------------------------------------------*/
size_t pkv_sample_workspace_bytes(int32_t num_rows, int32_t vocab_size);
int pkv_sample(int32_t* tokens, const void* logits, int64_t row_stride, int32_t num_rows,
               int32_t vocab_size, pkv_dtype_t dtype, const float* temperatures, uint64_t seed,
               uint64_t offset, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Host block manager with prefix caching - [P1] Block, BlockManager and Sequence listings
 * and the Scheduler that calls them (schedule, preempt, postprocess); [P2] 请求执行 –
 * 输入序列预处理与context构建 for what the tables and cached counts feed. Host memory only;
 * nothing here touches the GPU. The manager owns its sequences (token ids, block table,
 * cached and scheduled token counts), addressed by the id pkv_bm_add_sequence returns.
 *
 * Hash of a block: XXH64 (seed 0, the published xxHash algorithm) over the previous block's
 * hash as 8 little-endian bytes (omitted for the first block, or when the previous block
 * carries no hash) followed by the block's token ids as 64-bit little-endian integers.
 * pkv_xxh64 and pkv_block_hash expose the two.
 *
 * Policy ([P1] BlockManager): free blocks sit on a FIFO; a used block's reference count is
 * the number of tables holding it. pkv_bm_can_allocate(seq) walks the sequence's full
 * blocks except its last, chaining the hash, while the index maps the hash to a block whose
 * token ids are equal: it returns the number of such cache hits, or -1 when the FIFO holds
 * fewer blocks than the table needs beyond its hits on used blocks. pkv_bm_allocate(seq, n)
 * fills an empty table: the first n hits reuse their blocks (a used block gains a
 * reference, a free one leaves the FIFO), the rest come off the FIFO's front (a block
 * handed out drops its hash from the index and forgets its contents); the cached token
 * count becomes n * block_size. pkv_bm_deallocate drops one reference per entry, last
 * entry first; blocks reaching zero join the FIFO's back and keep their hash until handed
 * out again. pkv_bm_can_append / pkv_bm_may_append: when the sequence's length is 1 modulo
 * block_size (its newest token opens a block), one more free block is needed / appended.
 * pkv_bm_set_scheduled records the step's token count (cached + scheduled <= length);
 * pkv_bm_hash_blocks seals the blocks that cached + scheduled tokens complete, chaining from
 * the previous block's hash, and indexes them; pkv_bm_commit_scheduled then adds the
 * scheduled count to the cached count (the engine's postprocess order).
 *
 * Returns: counts or ids >= 0 where stated, else PKV_OK; PKV_ERR_INVALID for a null
 * handle, an unknown or removed sequence id, a non-empty table for can_allocate / allocate,
 * hits that are no longer hits or a FIFO too short for allocate, an empty FIFO for
 * may_append, counts out of range, block_size < 2 or num_blocks < 1 for create.
 * pkv_bm_block_table / pkv_bm_free_block_ids copy up to `capacity` ids and return the full
 * count. pkv_bm_remove_sequence forgets a sequence whose table is empty.
 * -------------------------------------------------------------------------------------*/
typedef struct pkv_block_manager pkv_block_manager;

uint64_t pkv_xxh64(const void* data, size_t len, uint64_t seed);
int pkv_block_hash(const int64_t* token_ids, int32_t num_tokens, int32_t has_prefix,
                   uint64_t prefix, uint64_t* hash_out);
int pkv_bm_create(pkv_block_manager** handle, int32_t num_blocks, int32_t block_size);
int pkv_bm_destroy(pkv_block_manager* handle);
int pkv_bm_add_sequence(pkv_block_manager* handle, const int64_t* token_ids, int32_t num_tokens);
int pkv_bm_append_token(pkv_block_manager* handle, int32_t seq, int64_t token_id);
int pkv_bm_can_allocate(const pkv_block_manager* handle, int32_t seq);
int pkv_bm_allocate(pkv_block_manager* handle, int32_t seq, int32_t num_cached_blocks);
int pkv_bm_deallocate(pkv_block_manager* handle, int32_t seq);
int pkv_bm_can_append(const pkv_block_manager* handle, int32_t seq);
int pkv_bm_may_append(pkv_block_manager* handle, int32_t seq);
int pkv_bm_set_scheduled(pkv_block_manager* handle, int32_t seq, int32_t num_scheduled_tokens);
int pkv_bm_hash_blocks(pkv_block_manager* handle, int32_t seq);
int pkv_bm_commit_scheduled(pkv_block_manager* handle, int32_t seq);
int pkv_bm_sequence_info(const pkv_block_manager* handle, int32_t seq, int64_t* num_tokens,
                         int64_t* num_cached_tokens, int64_t* num_scheduled_tokens,
                         int32_t* table_len);
int pkv_bm_block_table(const pkv_block_manager* handle, int32_t seq, int32_t* out,
                       int32_t capacity);
int pkv_bm_num_free_blocks(const pkv_block_manager* handle);
int pkv_bm_free_block_ids(const pkv_block_manager* handle, int32_t* out, int32_t capacity);
int pkv_bm_block_info(const pkv_block_manager* handle, int32_t block_id, int32_t* ref_count,
                      int32_t* sealed, uint64_t* hash);
int pkv_bm_remove_sequence(pkv_block_manager* handle, int32_t seq);

#ifdef __cplusplus
}
#endif
#endif /* PAGED_KV_H_ */
