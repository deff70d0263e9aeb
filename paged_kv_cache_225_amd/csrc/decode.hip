// Paged decode attention with a split-K softmax, for gfx950.
//
// The operation is the decode branch of Attention.forward in "vLLM 学习笔记 02：nano-vllm
// 源码逐段精读": one query per sequence attends every cached key of the sequence (context
// length = len(seq), newest token included), K/V gathered through the block table.
//
// Work unit of decode_partial_kernel: (partition p, kv head g, sequence b). The unit reads
// the K and V rows of its keys for kv head g only and serves all G query heads of the
// group, so each K/V byte is read from HBM once. Inside a workgroup (4 wavefronts):
//   * a K or V row of one head (D elements) is spread over LPR lanes, 16 bytes per lane,
//     so one wavefront load instruction reads RPI whole rows;
//   * pass 1 loads K in chunks of kNI instructions per wave (kNI loads in flight per lane),
//     forms the G dot products per row with a DPP reduction inside the row's lanes and
//     leaves the scaled scores (log2 units) in LDS;
//   * pass 2 takes the partition's max and sum of exp2 over the LDS scores;
//   * pass 3 loads V the same way and accumulates the weighted rows in registers, then
//     reduces across the rows of a wavefront (shuffles) and across wavefronts (LDS).
// A sequence with a single partition writes its output directly; otherwise the unit
// writes (max, sum, weighted V) for each head and decode_reduce_kernel combines them:
//   M = max_p m_p, L = sum_p 2^(m_p - M) l_p, out = sum_p 2^(m_p - M) o_p / L.
// Keys past the context length are never loaded: block-table padding and the unused
// (possibly NaN) slots of a sequence's last block are not touched.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace pkv {

constexpr int kNI = 8;  // load instructions per wavefront per chunk

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    T* __restrict__ out, const T* __restrict__ q, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, int32_t num_blocks, const int32_t* __restrict__ block_tables,
    int32_t bt_stride, const int32_t* __restrict__ context_lens, int32_t num_kv_heads,
    int32_t bs_log2, float scale_log2e, int32_t part, int32_t max_parts,
    float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  using E = Elem<T>;
  constexpr int EPL = E::kPerChunk;  // elements per 16-byte lane chunk
  constexpr int LPR = D / EPL;       // lanes per row
  constexpr int RPI = 64 / LPR;      // rows per wavefront instruction
  constexpr int CH = 4 * RPI * kNI;  // keys per chunk (workgroup)
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row must tile a wavefront");

  __shared__ float s_sc[G][kDecodeMaxPartition];
  __shared__ float s_red[4][G];
  __shared__ float s_o[4][G][D];

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hq = num_kv_heads * G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, rsub = lane / LPR;

  int n = context_lens[b];
  const int cap = bt_stride << bs_log2;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int nparts = (n + part - 1) / part;
  T* out_bg = out + ((int64_t)b * Hq + (int64_t)g * G) * D;
  if (n == 0) {
    if (p == 0)
      for (int i = threadIdx.x; i < G * D; i += 256) E::store(out_bg + i, 0.f);
    return;
  }
  if (p >= nparts) return;
  const int k0 = p * part;
  const int nk = min(part, n - k0);

  const int64_t row_elems = (int64_t)num_kv_heads * D;
  const int64_t head_off = (int64_t)g * D + sub * EPL;
  const int32_t* bt = block_tables + (int64_t)b * bt_stride;
  const int bs_mask = (1 << bs_log2) - 1;

  float qf[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
    E::unpack(load16(q + ((int64_t)b * Hq + g * G + h) * D + sub * EPL), qf[h]);

  auto load_rows = [&](const T* cache, int c0, u32x4_t* r) {
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const int kl = c0 + (wave * kNI + i) * RPI + rsub;
      r[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (kl < nk) {
        const int j = k0 + kl;
        const int blk = bt[j >> bs_log2];
        if ((unsigned)blk < (unsigned)num_blocks)
          r[i] = load16(cache + (((int64_t)blk << bs_log2) + (j & bs_mask)) * row_elems + head_off);
        else
          r[i] = E::nan_chunk();
      }
    }
  };

  // ---- pass 1: scores -------------------------------------------------------------------
  for (int c0 = 0; c0 < nk; c0 += CH) {
    u32x4_t kr[kNI];
    load_rows(k_cache, c0, kr);
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      float kf[EPL];
      E::unpack(kr[i], kf);
      const int kl = c0 + (wave * kNI + i) * RPI + rsub;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(qf[h][e], kf[e], s);
        s = group_sum<LPR>(s);
        if (sub == 0 && kl < nk) s_sc[h][kl] = s * scale_log2e;
      }
    }
  }
  __syncthreads();

  // ---- pass 2: partition max and sum of exp2 -------------------------------------------
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = -INFINITY;
    for (int t = threadIdx.x; t < nk; t += 256) mx = fmaxf(mx, s_sc[h][t]);
    mx = group_max<64>(mx);
    if (lane == 0) s_red[wave][h] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h)
    m[h] = fmaxf(fmaxf(s_red[0][h], s_red[1][h]), fmaxf(s_red[2][h], s_red[3][h]));
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float sum = 0.f;
    for (int t = threadIdx.x; t < nk; t += 256) {
      const float e = __builtin_amdgcn_exp2f(s_sc[h][t] - m[h]);
      s_sc[h][t] = e;
      sum += e;
    }
    sum = group_sum<64>(sum);
    if (lane == 0) s_red[wave][h] = sum;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) l[h] = (s_red[0][h] + s_red[1][h]) + (s_red[2][h] + s_red[3][h]);

  // ---- pass 3: weighted V ----------------------------------------------------------------
  float o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  for (int c0 = 0; c0 < nk; c0 += CH) {
    u32x4_t vr[kNI];
    load_rows(v_cache, c0, vr);
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const int kl = c0 + (wave * kNI + i) * RPI + rsub;
      if (kl < nk) {
        float vf[EPL];
        E::unpack(vr[i], vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pw = s_sc[h][kl];
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(pw, vf[e], o[h][e]);
        }
      }
    }
  }
  // rows of one wavefront -> lanes 0..LPR-1
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e)
#pragma unroll
      for (int msk = LPR; msk < 64; msk <<= 1) o[h][e] += __shfl_xor(o[h][e], msk);
  if (rsub == 0)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][h][sub * EPL + e] = o[h][e];
  __syncthreads();

  for (int i = threadIdx.x; i < G * D; i += 256) {
    const int h = i / D, d = i % D;
    const float acc = (s_o[0][h][d] + s_o[1][h][d]) + (s_o[2][h][d] + s_o[3][h][d]);
    if (nparts == 1) {
      E::store(out_bg + i, acc / l[h]);
    } else {
      const int64_t u = ((int64_t)b * Hq + g * G + h) * max_parts + p;
      ws_o[u * D + d] = acc;
      if (d == 0) {
        ws_ml[2 * u] = m[h];
        ws_ml[2 * u + 1] = l[h];
      }
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(
    T* __restrict__ out, const int32_t* __restrict__ context_lens, int32_t cap, int32_t Hq,
    int32_t part, int32_t max_parts, const float* __restrict__ ws_o,
    const float* __restrict__ ws_ml) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  int n = context_lens[b];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int nparts = (n + part - 1) / part;
  if (nparts <= 1) return;
  const int64_t base = ((int64_t)b * Hq + h) * max_parts;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ws_ml[2 * (base + p)]);
  float L = 0.f, acc = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = __builtin_amdgcn_exp2f(ws_ml[2 * (base + p)] - M);
    L = fmaf(w, ws_ml[2 * (base + p) + 1], L);
    acc = fmaf(w, ws_o[(base + p) * D + d], acc);
  }
  Elem<T>::store(out + ((int64_t)b * Hq + h) * D + d, acc / L);
}

template <typename T, int D, int G>
static int run_decode(const DecodeArgs& a, hipStream_t stream) {
  const int bs_log2 = __builtin_ctz((unsigned)a.block_size);
  const float c = a.scale * kLog2e;
  dim3 grid1(a.max_parts, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partial_kernel<T, D, G>), grid1, dim3(256), 0, stream, (T*)a.out,
                     (const T*)a.q, (const T*)a.k_cache, (const T*)a.v_cache, a.num_blocks,
                     a.block_tables, a.max_blocks_per_seq, a.context_lens, a.num_kv_heads,
                     bs_log2, c, a.partition, a.max_parts, a.ws_o, a.ws_ml);
  if (a.max_parts > 1) {
    dim3 grid2(a.num_heads, a.num_seqs);
    hipLaunchKernelGGL((decode_reduce_kernel<T, D>), grid2, dim3(D), 0, stream, (T*)a.out,
                       a.context_lens, a.max_blocks_per_seq * a.block_size, a.num_heads,
                       a.partition, a.max_parts, a.ws_o, a.ws_ml);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

template <typename T, int D>
static int dispatch_g(const DecodeArgs& a, hipStream_t s) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return run_decode<T, D, 1>(a, s);
    case 2: return run_decode<T, D, 2>(a, s);
    case 4: return run_decode<T, D, 4>(a, s);
    case 8: return run_decode<T, D, 8>(a, s);
    default: return -2;
  }
}

int launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return 0;
  if (a.bf16) {
    if (a.head_dim == 128) return dispatch_g<__bf16, 128>(a, stream);
    if (a.head_dim == 64) return dispatch_g<__bf16, 64>(a, stream);
  } else {
    if (a.head_dim == 128) return dispatch_g<float, 128>(a, stream);
    if (a.head_dim == 64) return dispatch_g<float, 64>(a, stream);
  }
  return -2;
}

}  // namespace pkv
