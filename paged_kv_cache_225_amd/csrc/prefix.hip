// Shared prefix blocks as a kernel of their own: the decode_prefix_unit work units (one
// shared block, a head group, up to 64 member sequences) on a 3-D grid, launched after the
// stream kernel. Used where the stream kernel's grid cannot take the units as extra
// workgroups (its register or LDS budget; see run_decode).
#include "prefix_unit.hpp"

namespace pkv {
namespace {

template <int D, int GH>
__global__ __launch_bounds__(256, 2) void decode_prefix_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k_cache,
    const __bf16* __restrict__ v_cache, int32_t num_blocks,
    const int32_t* __restrict__ block_tables, int32_t bt_stride,
    const int32_t* __restrict__ g_ptr, const int32_t* __restrict__ g_members,
    const int32_t* __restrict__ g_col, int32_t num_heads, int32_t num_kv_heads,
    int32_t bs_log2, float scale_log2e, float* __restrict__ pfx_o, float* __restrict__ pfx_ml) {
  decode_prefix_unit<D, GH>(blockIdx.x, blockIdx.y, blockIdx.z, q, k_cache, v_cache, num_blocks,
                            block_tables, bt_stride, g_ptr, g_members, g_col, num_heads,
                            num_kv_heads, bs_log2, scale_log2e, pfx_o, pfx_ml);
}

template <int D, int GH>
int run_prefix(const PrefixArgs& a, hipStream_t stream) {
  dim3 grid(a.num_heads / GH, a.num_groups, (a.max_group_size + 63) / 64);
  hipLaunchKernelGGL((decode_prefix_kernel<D, GH>), grid, dim3(256), 0, stream,
                     (const __bf16*)a.q, (const __bf16*)a.k_cache, (const __bf16*)a.v_cache,
                     a.num_blocks, a.block_tables, a.max_blocks_per_seq, a.group_ptr,
                     a.group_members, a.group_col, a.num_heads, a.num_kv_heads,
                     __builtin_ctz((unsigned)a.block_size), a.scale * kLog2e, a.pfx_o, a.pfx_ml);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

int launch_decode_prefix(const PrefixArgs& a, hipStream_t stream) {
  if (a.num_groups == 0 || a.max_group_size == 0) return 0;
  const bool pair = (a.num_heads / a.num_kv_heads) % 2 == 0;
  if (a.head_dim == 128) return pair ? run_prefix<128, 2>(a, stream) : run_prefix<128, 1>(a, stream);
  if (a.head_dim == 64) return pair ? run_prefix<64, 2>(a, stream) : run_prefix<64, 1>(a, stream);
  return -2;
}

}  // namespace pkv
