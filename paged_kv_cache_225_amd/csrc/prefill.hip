// Varlen causal prefill attention over the paged cache, for gfx950 (bf16 MFMA).
//
// The operation is the prefill branch of Attention.forward in "vLLM 学习笔记 02：nano-vllm
// 源码逐段精读" (flash_attn_varlen_func with a block table): sequence b has Lq packed query
// rows and Lk >= Lq keys; query i sits at position Lk - Lq + i and sees keys up to it, so
// cached-prefix keys ("Nano-vLLM代码手撕笔记", 请求执行 – 输入序列预处理与context构建: Q=[CDEF],
// K=[ABCDEF]) are visible to every query.
//
// Work unit: (q-head group of GH heads sharing one kv head, sequence b, 64 query positions).
// Units are numbered from the end of each sequence so the longest rows (most keys) are
// dispatched first. Each of the 4 wavefronts owns 16 query positions x GH heads.
//
// Per key tile of 64 keys, staged through LDS (K row-major, V transposed):
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 dims of K (one 16-byte LDS
//                 read per lane), B = Q^T held in registers for the whole unit. The result
//                 leaves lane l with 4 keys of query column l % 16, so the running max, the
//                 exp2 and the running sum stay per lane (two cross-lane steps per tile for
//                 the max only).
//   O^T += V^T P^T  with the same MFMA: the B operand is the lane's own probabilities
//                 (bf16), the A operand reads V^T from LDS with the key order that matches
//                 the lane's registers. O^T accumulates in registers, one query per lane.
// The softmax is the online form: m' = max(m, tile max), O and l scaled by 2^(m - m').
// Scores enter exp2 as s * scale * log2(e). Keys past Lk are zero-filled in LDS (never
// read from the cache), so padding entries and unused NaN slots cannot reach an MFMA.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace pkv {

constexpr int kBK = 64;  // keys per tile
constexpr int kBQ = 64;  // query positions per workgroup

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int GH>
__global__ __launch_bounds__(256) void prefill_kernel(
    __bf16* __restrict__ out, const __bf16* __restrict__ q, const __bf16* __restrict__ k_cache,
    const __bf16* __restrict__ v_cache, int32_t num_blocks,
    const int32_t* __restrict__ block_tables, int32_t bt_stride,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int32_t num_heads,
    int32_t num_kv_heads, int32_t bs_log2, float scale_log2e) {
  constexpr int KS = D / 32;             // k-steps of the QK^T product
  constexpr int DT = D / 16;             // 16-row tiles of O^T
  constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
  constexpr int NC = kBK * CPR / 256;    // chunks per thread per tile
  constexpr int KSTR = D + 8;            // K tile row stride (elements)
  constexpr int VSTR = kBK + 4;          // V^T tile row stride (elements)
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kBK * KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[D * VSTR];

  const int hg = blockIdx.x, b = blockIdx.y, t = blockIdx.z;
  const int G = num_heads / num_kv_heads;
  const int h0 = hg * GH, g = h0 / G;
  const int q_begin = cu_q[b];
  const int Lq = cu_q[b + 1] - q_begin;
  const int cap = bt_stride << bs_log2;
  int Lk = cu_k[b + 1] - cu_k[b];
  Lk = Lk > cap ? cap : Lk;
  const int i_hi = Lq - kBQ * t;  // exclusive end of this unit's query rows
  if (i_hi <= 0) return;
  const int i_lo = i_hi - kBQ;    // may be negative: those rows are idle
  const int off = Lk - Lq;        // position of query row 0

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int i_row = i_lo + wave * 16 + col;
  const bool row_ok = i_row >= 0;
  const int pos = off + i_row;
  const int kend = min(Lk, off + i_hi);
  const int n_kt = kend > 0 ? (kend + kBK - 1) / kBK : 0;
  const int wave_min_pos = off + i_lo + wave * 16;

  const int64_t row_elems = (int64_t)num_kv_heads * D;
  const int32_t* bt = block_tables + (int64_t)b * bt_stride;
  const int bs_mask = (1 << bs_log2) - 1;

  // Q^T operands: lane holds 8 dims of its query column for each k-step
  bf16x8_t qb[GH][KS];
#pragma unroll
  for (int nt = 0; nt < GH; ++nt)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (row_ok)
        v = load16(q + ((int64_t)(q_begin + i_row) * num_heads + h0 + nt) * D + 32 * s + 8 * quad);
      qb[nt][s] = __builtin_bit_cast(bf16x8_t, v);
    }

  f32x4_t oacc[DT][GH];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int nt = 0; nt < GH; ++nt) oacc[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[GH], l_run[GH];
#pragma unroll
  for (int nt = 0; nt < GH; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }

  u32x4_t kreg[NC], vreg[NC];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int u = i * 256 + tid;
      const int key = u / CPR, c = u % CPR;
      const int j = kt * kBK + key;
      kreg[i] = u32x4_t{0u, 0u, 0u, 0u};
      vreg[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (j < Lk) {
        const int blk = bt[j >> bs_log2];
        if ((unsigned)blk < (unsigned)num_blocks) {
          const int64_t o = (((int64_t)blk << bs_log2) + (j & bs_mask)) * row_elems +
                            (int64_t)g * D + 8 * c;
          kreg[i] = load16(k_cache + o);
          vreg[i] = load16(v_cache + o);
        } else {
          kreg[i] = Elem<__bf16>::nan_chunk();
          vreg[i] = Elem<__bf16>::nan_chunk();
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int u = i * 256 + tid;
      const int key = u / CPR, c = u % CPR;
      store16(&Ks[key * KSTR + 8 * c], kreg[i]);
      const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(8 * c + 2 * e) * VSTR + key] = __builtin_bit_cast(__bf16, (uint16_t)(w[e] & 0xffffu));
        Vt[(8 * c + 2 * e + 1) * VSTR + key] = __builtin_bit_cast(__bf16, (uint16_t)(w[e] >> 16));
      }
    }
  };

  if (n_kt > 0) load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(kt + 1);

    // S^T = K Q^T : sacc[mt][nt][r] = score of key kt*64 + 16 mt + 4 quad + r, column col
    f32x4_t sacc[4][GH];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < GH; ++nt) sacc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&Ks[(16 * mt + col) * KSTR + 32 * s + 8 * quad]);
#pragma unroll
        for (int nt = 0; nt < GH; ++nt) sacc[mt][nt] = mfma16(a, qb[nt][s], sacc[mt][nt]);
      }

    const bool need_mask = kt * kBK + kBK - 1 > wave_min_pos;
    bf16x8_t pb[2][GH];
#pragma unroll
    for (int nt = 0; nt < GH; ++nt) {
      float sv[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float s = sacc[mt][nt][r];
          if (need_mask) {
            const int j = kt * kBK + 16 * mt + 4 * quad + r;
            s = (j <= pos) ? s : -INFINITY;
          }
          sv[mt][r] = s;
          mx = fmaxf(mx, s);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run[nt] - m_use) * scale_log2e);
      const float mc = m_use * scale_log2e;
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sv[mt][r], scale_log2e, -mc));
          sv[mt][r] = e;
          psum += e;
        }
      l_run[nt] = fmaf(alpha, l_run[nt], psum);
      m_run[nt] = m_new;
#pragma unroll
      for (int i = 0; i < DT; ++i) oacc[i][nt] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t w;
        w.x = pack_bf16x2(sv[2 * ks][0], sv[2 * ks][1]);
        w.y = pack_bf16x2(sv[2 * ks][2], sv[2 * ks][3]);
        w.z = pack_bf16x2(sv[2 * ks + 1][0], sv[2 * ks + 1][1]);
        w.w = pack_bf16x2(sv[2 * ks + 1][2], sv[2 * ks + 1][3]);
        pb[ks][nt] = __builtin_bit_cast(bf16x8_t, w);
      }
    }

    // O^T += V^T P^T ; A operand lane (row d = 16 i + col) holds keys
    // {32 ks + 4 quad + 0..3} then {32 ks + 16 + 4 quad + 0..3}, matching pb's order.
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const __bf16* vrow = &Vt[(16 * i + col) * VSTR + 32 * ks + 4 * quad];
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 16);
        const u32x4_t w = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
        for (int nt = 0; nt < GH; ++nt) oacc[i][nt] = mfma16(a, pb[ks][nt], oacc[i][nt]);
      }
  }

  // normalise and store: lane holds dims 16 i + 4 quad + r of its query column
#pragma unroll
  for (int nt = 0; nt < GH; ++nt) {
    float l = l_run[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.f / l;
    if (row_ok) {
      __bf16* orow = out + ((int64_t)(q_begin + i_row) * num_heads + h0 + nt) * D;
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        u32x2_t w;
        w.x = pack_bf16x2(oacc[i][nt][0] * inv, oacc[i][nt][1] * inv);
        w.y = pack_bf16x2(oacc[i][nt][2] * inv, oacc[i][nt][3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + 16 * i + 4 * quad) = w;
      }
    }
  }
}

template <int D, int GH>
static int run_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int bs_log2 = __builtin_ctz((unsigned)a.block_size);
  const int n_tiles = (a.max_seqlen_q + kBQ - 1) / kBQ;
  dim3 grid(a.num_heads / GH, a.num_seqs, n_tiles);
  hipLaunchKernelGGL((prefill_kernel<D, GH>), grid, dim3(256), 0, stream, (__bf16*)a.out,
                     (const __bf16*)a.q, (const __bf16*)a.k_cache, (const __bf16*)a.v_cache,
                     a.num_blocks, a.block_tables, a.max_blocks_per_seq, a.cu_seqlens_q,
                     a.cu_seqlens_k, a.num_heads, a.num_kv_heads, bs_log2,
                     a.scale * kLog2e);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_seqlen_q == 0) return 0;
  const int G = a.num_heads / a.num_kv_heads;
  const bool pair = (G % 2) == 0;
  if (a.head_dim == 128) return pair ? run_prefill<128, 2>(a, stream) : run_prefill<128, 1>(a, stream);
  if (a.head_dim == 64) return pair ? run_prefill<64, 2>(a, stream) : run_prefill<64, 1>(a, stream);
  return -2;
}

}  // namespace pkv
