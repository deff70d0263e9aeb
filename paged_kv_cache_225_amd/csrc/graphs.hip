// Decode steps replayed from captured HIP graphs, one graph per batch bucket.
//
// The engine in "vLLM 学习笔记 02：nano-vllm 源码逐段精读" (ModelRunner.capture_cudagraph and
// run_model) records the decode step once per batch size of a fixed list (1, 2, 4, 8, then
// every multiple of 16 up to the largest batch) over static buffers sized for the largest
// batch; a step of batch B fills the first B rows of those buffers, pads the rest (slot -1,
// context length 0) and replays the graph of the smallest recorded batch >= B. "Nano-vLLM代码
// 手撕笔记" (cuda graph捕捉与context设置) gives the reason: the shapes and device addresses a
// graph records are fixed, and one launch of the graph replaces the step's kernel launches.
//
// Here each graph holds, for every attention layer of the model, one paged_attn_decode_store
// call (the decode kernels with the store fused in) at that bucket's row count: the engine's
// graph covers the whole forward, so one launch replaces the launches of every layer.
// Layers have their own pools and rows but share the step's metadata (slot_mapping, block
// tables, context lengths), as all layers of that model read one Context. The launch configuration depends only on the row
// count and the static table width, and everything that depends on the data (shares of the
// split, piece counts) is computed on the device from context_lens at run time, so a
// recorded call stays correct for any lengths written into the buffers before a replay.
// Nothing is allocated on the device and no memset is recorded.
#include <stdint.h>
#include <stdlib.h>

#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "paged_kv.h"

struct pkv_decode_graphs {
  int32_t max_batch = 0;
  int32_t num_layers = 0;
  std::vector<int32_t> buckets;     // ascending
  std::vector<hipGraph_t> graphs;   // one per bucket
  std::vector<hipGraphExec_t> execs;
};

namespace {

void release(pkv_decode_graphs* g) {
  if (!g) return;
  for (hipGraphExec_t e : g->execs)
    if (e) (void)hipGraphExecDestroy(e);
  for (hipGraph_t gr : g->graphs)
    if (gr) (void)hipGraphDestroy(gr);
  delete g;
}

// 1, 2, 4, 8, then 16, 32, ... up to max_batch; max_batch itself is appended when it is not
// on that list, so that every batch up to max_batch has a bucket.
std::vector<int32_t> bucket_list(int32_t max_batch) {
  std::vector<int32_t> v;
  for (int32_t b : {1, 2, 4, 8})
    if (b <= max_batch) v.push_back(b);
  for (int32_t b = 16; b <= max_batch; b += 16) v.push_back(b);
  if (v.empty() || v.back() != max_batch) v.push_back(max_batch);
  return v;
}

int bucket_index(const pkv_decode_graphs* g, int32_t batch) {
  if (!g || batch < 1 || batch > g->max_batch) return -1;
  for (size_t i = 0; i < g->buckets.size(); ++i)
    if (g->buckets[i] >= batch) return (int)i;
  return -1;
}

}  // namespace

extern "C" {

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
                                    void* workspace, size_t workspace_bytes) {
  if (!handle) return PKV_ERR_INVALID;
  *handle = nullptr;
  if (max_batch < 1 || max_batch > 16383) return PKV_ERR_INVALID;
  if (num_layers < 1 || num_layers > 1024) return PKV_ERR_INVALID;
  if (!out || !q || !key || !value || !k_cache || !v_cache) return PKV_ERR_INVALID;
  const size_t need = paged_attn_decode_workspace_bytes(max_batch, num_heads, head_dim,
                                                        max_blocks_per_seq, block_size,
                                                        partition_size);
  if (need == 0) return PKV_ERR_INVALID;
  if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;

  pkv_decode_graphs* g = new (std::nothrow) pkv_decode_graphs;
  if (!g) return PKV_ERR_HIP;
  g->max_batch = max_batch;
  g->num_layers = num_layers;
  g->buckets = bucket_list(max_batch);

  hipStream_t cs = nullptr;  // a private stream to record on (default priority)
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) {
    release(g);
    return PKV_ERR_HIP;
  }
  int rc = PKV_OK;
  // the engine records the largest batch first; the order does not matter here
  for (size_t i = 0; i < g->buckets.size() && rc == PKV_OK; ++i) {
    const int32_t bs = g->buckets[i];
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      rc = PKV_ERR_HIP;
      break;
    }
    int call = PKV_OK;
    for (int32_t l = 0; l < num_layers && call == PKV_OK; ++l)
      call = paged_attn_decode_store(
          out[l], q[l], key[l], key_token_stride, value[l], value_token_stride, slot_mapping,
          k_cache[l], v_cache[l], num_blocks, block_tables, max_blocks_per_seq, context_lens,
          bs, num_heads, num_kv_heads, head_dim, block_size, scale, dtype, partition_size,
          kv_stream_from, workspace, workspace_bytes, cs);
    const hipError_t end = hipStreamEndCapture(cs, &graph);
    if (call != PKV_OK || end != hipSuccess || !graph) {
      if (graph) (void)hipGraphDestroy(graph);
      rc = call != PKV_OK ? call : PKV_ERR_HIP;
      break;
    }
    g->graphs.push_back(graph);
    hipGraphExec_t exec = nullptr;
    if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess || !exec) {
      rc = PKV_ERR_HIP;
      break;
    }
    g->execs.push_back(exec);
  }
  (void)hipStreamDestroy(cs);
  if (rc != PKV_OK) {
    (void)hipGetLastError();  // the error is reported through the status
    release(g);
    return rc;
  }
  *handle = g;
  return PKV_OK;
}

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
                             void* workspace, size_t workspace_bytes) {
  return pkv_decode_graphs_create_layers(
      handle, max_batch, 1, &out, &q, &key, key_token_stride, &value, value_token_stride,
      slot_mapping, &k_cache, &v_cache, num_blocks, block_tables, max_blocks_per_seq,
      context_lens, num_heads, num_kv_heads, head_dim, block_size, scale, dtype,
      partition_size, kv_stream_from, workspace, workspace_bytes);
}

int pkv_decode_graphs_count(const pkv_decode_graphs* g) {
  return g ? (int)g->buckets.size() : PKV_ERR_INVALID;
}

int pkv_decode_graphs_buckets(const pkv_decode_graphs* g, int32_t* buckets, int32_t capacity) {
  if (!g || (!buckets && capacity > 0) || capacity < 0) return PKV_ERR_INVALID;
  const int n = (int)g->buckets.size();
  for (int i = 0; i < n && i < capacity; ++i) buckets[i] = g->buckets[i];
  return n;
}

int pkv_decode_graphs_bucket(const pkv_decode_graphs* g, int32_t batch) {
  const int i = bucket_index(g, batch);
  return i < 0 ? PKV_ERR_INVALID : g->buckets[i];
}

int pkv_decode_graphs_launch(pkv_decode_graphs* g, int32_t batch, hipStream_t stream) {
  const int i = bucket_index(g, batch);
  if (i < 0) return PKV_ERR_INVALID;
  if (hipGraphLaunch(g->execs[i], stream) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}

int pkv_decode_graphs_destroy(pkv_decode_graphs* g) {
  if (!g) return PKV_ERR_INVALID;
  release(g);
  return PKV_OK;
}

}  // extern "C"
