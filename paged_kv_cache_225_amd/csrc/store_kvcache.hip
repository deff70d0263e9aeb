// K/V slot scatter for gfx950.
//
// Follows the store_kvcache listing of "vLLM 学习笔记 02：nano-vllm 源码逐段精读": token t's
// key and value rows (all kv heads, Hkv*D contiguous elements) are copied into cache slot
// slot_mapping[t]; slot -1 skips the token. The copy is bitwise.
//
// Layout of the work: one thread per 16-byte chunk, chunks ordered token-major, K row then
// V row, so consecutive lanes read and write consecutive bytes of the same row (each
// wavefront instruction moves 1 KiB of one row). A grid-stride loop caps the launch size.
// Rows that are not 16-byte aligned (an odd token stride or base) take an element loop.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

__global__ __launch_bounds__(256) void store_kv_vec_kernel(
    const char* __restrict__ key, int64_t key_stride_bytes,
    const char* __restrict__ value, int64_t value_stride_bytes,
    char* __restrict__ k_cache, char* __restrict__ v_cache, int64_t num_slots,
    const int32_t* __restrict__ slot_mapping, int64_t num_tokens, int32_t row_chunks) {
  const int64_t per_token = 2 * (int64_t)row_chunks;
  const int64_t total = num_tokens * per_token;
  const int64_t row_bytes = (int64_t)row_chunks * 16;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / per_token;
    const int32_t r = (int32_t)(idx - t * per_token);
    const int32_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    const bool is_v = r >= row_chunks;
    const int32_t c = is_v ? r - row_chunks : r;
    const char* src = is_v ? value + t * value_stride_bytes : key + t * key_stride_bytes;
    char* dst = (is_v ? v_cache : k_cache) + (int64_t)slot * row_bytes;
    store16(dst + 16 * (int64_t)c, load16(src + 16 * (int64_t)c));
  }
}

template <typename W>
__global__ __launch_bounds__(256) void store_kv_elem_kernel(
    const W* __restrict__ key, int64_t key_stride, const W* __restrict__ value,
    int64_t value_stride, W* __restrict__ k_cache, W* __restrict__ v_cache, int64_t num_slots,
    const int32_t* __restrict__ slot_mapping, int64_t num_tokens, int32_t row_elems) {
  const int64_t per_token = 2 * (int64_t)row_elems;
  const int64_t total = num_tokens * per_token;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / per_token;
    const int32_t r = (int32_t)(idx - t * per_token);
    const int32_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    const bool is_v = r >= row_elems;
    const int32_t e = is_v ? r - row_elems : r;
    const W* src = is_v ? value + t * value_stride : key + t * key_stride;
    W* dst = (is_v ? v_cache : k_cache) + (int64_t)slot * row_elems;
    dst[e] = src[e];
  }
}

static unsigned grid_for(int64_t work) {
  int64_t blocks = (work + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  return (unsigned)(blocks < 1 ? 1 : blocks);
}

int launch_store_kvcache(const void* key, int64_t key_stride, const void* value,
                         int64_t value_stride, void* k_cache, void* v_cache, int64_t num_slots,
                         const int32_t* slot_mapping, int32_t num_tokens, int32_t row_elems,
                         int32_t elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return 0;
  const int64_t row_bytes = (int64_t)row_elems * elem_bytes;
  const int64_t ks = key_stride * elem_bytes, vs = value_stride * elem_bytes;
  const bool aligned = (row_bytes % 16 == 0) && (ks % 16 == 0) && (vs % 16 == 0) &&
                       ((uintptr_t)key % 16 == 0) && ((uintptr_t)value % 16 == 0) &&
                       ((uintptr_t)k_cache % 16 == 0) && ((uintptr_t)v_cache % 16 == 0);
  if (aligned) {
    const int32_t row_chunks = (int32_t)(row_bytes / 16);
    hipLaunchKernelGGL(store_kv_vec_kernel, dim3(grid_for((int64_t)num_tokens * 2 * row_chunks)),
                       dim3(256), 0, stream, (const char*)key, ks, (const char*)value, vs,
                       (char*)k_cache, (char*)v_cache, num_slots, slot_mapping,
                       (int64_t)num_tokens, row_chunks);
  } else if (elem_bytes == 4) {
    hipLaunchKernelGGL(store_kv_elem_kernel<uint32_t>,
                       dim3(grid_for((int64_t)num_tokens * 2 * row_elems)), dim3(256), 0, stream,
                       (const uint32_t*)key, key_stride, (const uint32_t*)value, value_stride,
                       (uint32_t*)k_cache, (uint32_t*)v_cache, num_slots, slot_mapping,
                       (int64_t)num_tokens, row_elems);
  } else {
    hipLaunchKernelGGL(store_kv_elem_kernel<uint16_t>,
                       dim3(grid_for((int64_t)num_tokens * 2 * row_elems)), dim3(256), 0, stream,
                       (const uint16_t*)key, key_stride, (const uint16_t*)value, value_stride,
                       (uint16_t*)k_cache, (uint16_t*)v_cache, num_slots, slot_mapping,
                       (int64_t)num_tokens, row_elems);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace pkv
