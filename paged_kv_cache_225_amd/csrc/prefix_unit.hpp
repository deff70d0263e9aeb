// Decode attention over shared prefix blocks, once per block for all the sequences sharing it
// (bf16 MFMA, gfx950).
//
// Prefix caching ("vLLM 学习笔记 02：nano-vllm 源码逐段精读", BlockManager: allocate reuses a
// cached block for every sequence whose token prefix hashes to it, so only leading full
// blocks are shared) makes many sequences of one decode step read the same physical blocks.
// The decode step's attention for query (sequence b, q head h) is
// softmax(scale q K^T) V over the sequence's keys; split by key ranges it is an exact merge
// of per-range partials (m, l, o): m the reference max, l = sum 2^(s - m), o = sum 2^(s - m) V,
// s in log2 units. decode_prefix_unit computes those partials for the key range of one
// shared block for every member sequence of a group (the sequences whose table holds that
// block in the same column), reading the block's K/V once per 64 members instead of once per
// member; the decode call's private keys go through the split-K stream kernel and the
// combine merges both. The units run as extra workgroups of the stream kernel's grid
// (decode_stream_prefix_kernel) or, where that grid cannot hold them, as their own kernel
// (prefix.hip).
//
// Work unit: (head group of GH q heads sharing one kv head, group g, 64 members). The 4
// wavefronts own 16 members x GH heads each - the prefill kernel's tile layout with members
// in place of query positions and no causal mask (every key of a shared block is visible).
// 64-key tiles go HBM -> LDS with buffer_load ... lds, double-buffered.
#pragma once

#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace pkv {
namespace {

constexpr int kPBK = 64;           // keys per tile
constexpr float kPSlack = 8.f;     // log2 units a tile max may exceed the reference max

// LDS of one unit: two stages of a K tile and a V tile, kPBK rows of D bf16 each
template <int D>
constexpr size_t kPrefixUnitLds = 2 * 2 * (size_t)kPBK * D * 2;
constexpr size_t kLdsPerCu = 160 * 1024;

typedef short ps16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) ps16x4_t plds_s16x4_t;

__device__ __forceinline__ f32x4_t pmfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max over lanes l, l^16, l^32, l^48 (VALU lane swaps)
__device__ __forceinline__ float prows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ void pwait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16 bytes per lane, base + voff bytes -> LDS at lds_base + 16 * lane (device pass only: the
// host pass must not see the builtins)
__device__ __forceinline__ void pload_lds16(const void* base, int voff, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
#endif
}

template <int D, int GH>
__device__ __forceinline__ void decode_prefix_unit(int hg, int g, int mc,
    const __bf16* __restrict__ q, const __bf16* __restrict__ k_cache,
    const __bf16* __restrict__ v_cache, int32_t num_blocks,
    const int32_t* __restrict__ block_tables, int32_t bt_stride,
    const int32_t* __restrict__ g_ptr, const int32_t* __restrict__ g_members,
    const int32_t* __restrict__ g_col, int32_t num_heads, int32_t num_kv_heads,
    int32_t bs_log2, float scale_log2e, float* __restrict__ pfx_o, float* __restrict__ pfx_ml) {
  constexpr int KS = D / 32;      // k-steps of the QK^T product
  constexpr int DT = D / 16;      // 16-row tiles of O^T
  constexpr int CPR = D / 8;      // 16-byte chunks per K/V row
  constexpr int RPL = 64 / CPR;   // rows per load instruction
  constexpr int NL = kPBK / RPL / 4;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = kPBK * ROWB;
  __shared__ __attribute__((aligned(1024))) char lds_a[2][TILEB];  // [K=0,V=1]
  __shared__ __attribute__((aligned(1024))) char lds_b[2][TILEB];
  static_assert(sizeof(lds_a) + sizeof(lds_b) == kPrefixUnitLds<D>, "unit LDS");

  const int m0 = g_ptr[g], n_mem = g_ptr[g + 1] - m0;
  if (mc * 64 >= n_mem) return;
  const int col_g = g_col[g];
  const int G = num_heads / num_kv_heads;
  const int h0 = hg * GH, kh = h0 / G;
  const int64_t row_elems = (int64_t)num_kv_heads * D;
  // every member holds the group's block in column col_g (a precondition); an id outside
  // the pool is never read: its keys become NaN, which poisons exactly the members' rows
  const int blk = block_tables[(int64_t)g_members[m0] * bt_stride + col_g];
  const bool blk_ok = (unsigned)blk < (unsigned)num_blocks;
  const int n_kt = (1 << bs_log2) / kPBK;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int mi = mc * 64 + wave * 16 + col;  // this lane's member (query column)
  const bool row_ok = mi < n_mem;
  const int b = row_ok ? g_members[m0 + mi] : 0;

  bf16x8_t qb[GH][KS];
#pragma unroll
  for (int nt = 0; nt < GH; ++nt)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (row_ok) v = load16(q + ((int64_t)b * num_heads + h0 + nt) * D + 32 * s + 8 * quad);
      qb[nt][s] = __builtin_bit_cast(bf16x8_t, v);
    }

  // load instruction i of this wave fills LDS bytes [(wave*NL + i) * 1024, +1024) of a tile:
  // rows RPL * (wave*NL + i) + lane / CPR; K chunks XOR-swizzled by the row in 16-byte units,
  // V in 32-byte units (conflict-free MFMA operand reads)
  const int slot = lane % CPR;
  int voff_k[NL], voff_v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int r = RPL * (wave * NL + i) + lane / CPR;
    const int kc = slot ^ (r % CPR);
    const int vc = 2 * ((slot >> 1) ^ (r % (CPR / 2))) + (slot & 1);
    voff_k[i] = 2 * (int)(r * row_elems + kh * D + 8 * kc);
    voff_v[i] = 2 * (int)(r * row_elems + kh * D + 8 * vc);
  }
  auto issue_tile = [&](int kt, char (*dst)[TILEB]) {
    if (blk_ok) {
      const int64_t base = (((int64_t)blk << bs_log2) + kt * kPBK) * row_elems;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        pload_lds16(k_cache + base, voff_k[i], &dst[0][(wave * NL + i) * 1024]);
        pload_lds16(v_cache + base, voff_v[i], &dst[1][(wave * NL + i) * 1024]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        store16(&dst[0][(wave * NL + i) * 1024] + 16 * lane, Elem<__bf16>::nan_chunk());
        store16(&dst[1][(wave * NL + i) * 1024] + 16 * lane, Elem<__bf16>::nan_chunk());
      }
    }
  };

  f32x4_t oacc[DT][GH];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int nt = 0; nt < GH; ++nt) oacc[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[GH];
  f32x4_t l_acc[GH];
#pragma unroll
  for (int nt = 0; nt < GH; ++nt) {
    m_run[nt] = -INFINITY;
    l_acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  issue_tile(0, lds_a);
  auto tile_step = [&](int kt, char (*cur)[TILEB], char (*nxt)[TILEB]) {
    pwait_vmem();
    __syncthreads();
    if (kt + 1 < n_kt) issue_tile(kt + 1, nxt);
    const char* Kt = cur[0];
    const char* Vt = cur[1];

    // S^T = K Q^T: sacc[mt][nt][r] = score of key kt*64 + 16 mt + 4 quad + r, column col
    f32x4_t sacc[4][GH];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < GH; ++nt) sacc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t ka[2][4];
    auto kread = [&](int s, int mt) {
      const int r = 16 * mt + col;
      const int c = (4 * s + quad) ^ (r % CPR);
      ka[s & 1][mt] = *reinterpret_cast<const bf16x8_t*>(Kt + r * ROWB + 16 * c);
    };
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) kread(0, mt);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (s + 1 < KS) kread(s + 1, mt);
#pragma unroll
        for (int nt = 0; nt < GH; ++nt) sacc[mt][nt] = pmfma(ka[s & 1][mt], qb[nt][s], sacc[mt][nt]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int s = 0; s + 1 < KS; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        __builtin_amdgcn_sched_group_barrier(0x008, GH, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * GH, 0);

    // online softmax (log2 units); the reference max moves only when a tile's max exceeds it
    // by more than kPSlack (or it is unset), so O is rarely rescaled
    bool need = false;
    float mxs[GH];
#pragma unroll
    for (int nt = 0; nt < GH; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[mt][nt][r]);
      mxs[nt] = prows_max(mx);
      need |= ((mxs[nt] - m_run[nt]) * scale_log2e > kPSlack) |
              ((m_run[nt] == -INFINITY) & (mxs[nt] != -INFINITY));
    }
    if (__any(need)) {
#pragma unroll
      for (int nt = 0; nt < GH; ++nt) {
        const float m_new = fmaxf(m_run[nt], mxs[nt]);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run[nt] - m_use) * scale_log2e);
        l_acc[nt] *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i) oacc[i][nt] *= alpha;
        m_run[nt] = m_new;
      }
    }
    float mcs[GH];
#pragma unroll
    for (int nt = 0; nt < GH; ++nt)
      mcs[nt] = (m_run[nt] == -INFINITY ? 0.f : m_run[nt]) * scale_log2e;
    bf16x8_t pb[2][GH];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nt = 0; nt < GH; ++nt) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          p[e] = __builtin_amdgcn_exp2f(
              fmaf(sacc[2 * ks + e / 4][nt][e % 4], scale_log2e, -mcs[nt]));
        u32x4_t w;
        w.x = pack_bf16x2(p[0], p[1]);
        w.y = pack_bf16x2(p[2], p[3]);
        w.z = pack_bf16x2(p[4], p[5]);
        w.w = pack_bf16x2(p[6], p[7]);
        pb[ks][nt] = __builtin_bit_cast(bf16x8_t, w);
      }

    // O^T += V^T P^T; lane (row d = 16 i + col, group quad) takes keys 32 ks + 4 quad + 0..3
    // and 32 ks + 16 + 4 quad + 0..3 through two transposing reads
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        ps16x4_t part[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int r = 32 * ks + 16 * hf + 4 * quad + (col >> 2);
          const int c2 = i ^ (r % (CPR / 2));
          const char* src = Vt + r * ROWB + 32 * c2 + 8 * (col & 3);
          part[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((plds_s16x4_t*)src);
        }
        u32x4_t w;
        w.x = __builtin_bit_cast(u32x2_t, part[0]).x;
        w.y = __builtin_bit_cast(u32x2_t, part[0]).y;
        w.z = __builtin_bit_cast(u32x2_t, part[1]).x;
        w.w = __builtin_bit_cast(u32x2_t, part[1]).y;
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
        for (int nt = 0; nt < GH; ++nt) oacc[i][nt] = pmfma(av, pb[ks][nt], oacc[i][nt]);
      }
    const bf16x8_t ones = __builtin_bit_cast(
        bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nt = 0; nt < GH; ++nt) l_acc[nt] = pmfma(ones, pb[ks][nt], l_acc[nt]);
  };
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile_step(kt, lds_a, lds_b);
    if (kt + 1 < n_kt) tile_step(kt + 1, lds_b, lds_a);
  }

  // partials of this block's keys: slot (b, h, column), o unnormalised, m in log2 units
  if (row_ok) {
#pragma unroll
    for (int nt = 0; nt < GH; ++nt) {
      const int64_t s = ((int64_t)b * num_heads + h0 + nt) * bt_stride + col_g;
      float* dst = pfx_o + s * D + 4 * quad;
#pragma unroll
      for (int i = 0; i < DT; ++i)
        store16(dst + 16 * i, u32x4_t{__float_as_uint(oacc[i][nt][0]), __float_as_uint(oacc[i][nt][1]),
                                      __float_as_uint(oacc[i][nt][2]), __float_as_uint(oacc[i][nt][3])});
      if (quad == 0) {
        pfx_ml[2 * s] = m_run[nt] * scale_log2e;
        pfx_ml[2 * s + 1] = l_acc[nt][0];
      }
    }
  }
}

}  // namespace
}  // namespace pkv
