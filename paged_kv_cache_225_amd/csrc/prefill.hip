// Varlen causal prefill attention over the paged cache, for gfx950 (bf16 MFMA).
//
// The operation is the prefill branch of Attention.forward in "vLLM 学习笔记 02：nano-vllm
// 源码逐段精读" (flash_attn_varlen_func with a block table): sequence b has Lq packed query
// rows and Lk >= Lq keys; query i sits at position Lk - Lq + i and sees keys up to it, so
// cached-prefix keys ("Nano-vLLM代码手撕笔记", 请求执行 – 输入序列预处理与context构建: Q=[CDEF],
// K=[ABCDEF]) are visible to every query.
//
// Work unit: (q-head group of GH heads sharing one kv head, sequence b, 64 query positions).
// Units are dispatched longest first (most 64-key tiles) so that short units fill the slots
// the long ones leave. Each of the 4 wavefronts owns 16 query positions x GH heads.
//
// Key tiles of 64 keys go from HBM straight into LDS with 16-byte buffer_load ... lds (no
// register staging), double-buffered: the loads of tile t+1 are issued right after the
// barrier that publishes tile t, and the block id of tile t+2 is looked up behind them (in
// a register window of the block table), so one barrier per tile is all the
// synchronisation there is. In LDS a K
// row keeps its 16-byte chunks XOR-swizzled by the row index and a V row its 32-byte
// chunks, so the MFMA operand reads below hit distinct banks.
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 dims of K (one ds_read_b128
//                 per lane, read one k-step ahead), B = Q^T held in registers for the
//                 whole unit. Lane l ends with
//                 4 keys of query column l % 16, so the running max, exp2 and the running sum
//                 stay per lane (two cross-lane steps per tile for the max).
//   O^T += V^T P^T  same MFMA: B = the lane's own probabilities (bf16); A = V^T, read with
//                 ds_read_b64_tr_b16, which hands every lane four consecutive keys of one
//                 head dimension - the key order the lane's probabilities are in.
// The softmax is the online form in log2 units: m' = max(m, tile max), O and l scaled by
// 2^(m - m') (skipped when no column's max moved). Keys past Lk are zero-filled in LDS and
// never read from the cache, so padding entries and unused NaN slots cannot reach an MFMA.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace pkv {

constexpr int kBK = 64;  // keys per tile
constexpr float kSlack = 8.f;  // log2 units a tile max may exceed the reference max
constexpr int kBQ = 64;  // query positions per workgroup

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Max over the four lanes l, l^16, l^32, l^48 (the 16-lane rows of a wavefront) with
// v_permlane16_swap / v_permlane32_swap: VALU lane exchanges, no LDS round trip.
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left free) through the builtin, so the compiler's own
// wait placement knows every earlier vector-memory result has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane (the
// small-block path, whose rows lie in different blocks: a lane's offset into the pool need
// not fit 32 bits). The builtin exists only for the device target; the host pass of this
// file must not see it (it would drop the kernels' launch stubs), so the body is compiled
// for the device pass only.
__device__ __forceinline__ void load_lds16(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
#endif
}

// The same through a buffer load (MUBUF) from the wave-uniform base + voff bytes (a tile
// inside one block, or packed rows: offsets of at most 63 rows). The global form is a
// FLAT-encoded instruction, and while one is in flight the compiler waits for every
// outstanding LDS read (lgkmcnt 0) wherever it needs one of them; with the buffer form it
// waits for just the reads it needs.
__device__ __forceinline__ void load_lds16_buf(const void* base, int voff, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
#endif
}

// BIG_BLOCKS: blocks hold >= 64 keys, so every 64-key tile lies inside one block.
// PACKED: no block table; sequence b's keys are rows cu_k[b] .. cu_k[b+1]-1 of k / v, with
// token strides k_stride / v_stride (elements). The paged form passes Hkv * D for both.
template <int D, int GH, bool BIG_BLOCKS, bool PACKED>
__global__ __launch_bounds__(256, 2) void prefill_kernel(
    __bf16* __restrict__ out, const __bf16* __restrict__ q, const __bf16* __restrict__ k_cache,
    const __bf16* __restrict__ v_cache, int32_t num_blocks,
    const int32_t* __restrict__ block_tables, int32_t bt_stride,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int32_t num_heads,
    int32_t num_kv_heads, int32_t bs_log2, float scale_log2e, int64_t k_stride,
    int64_t v_stride) {
  static_assert(BIG_BLOCKS || !PACKED, "packed rows take the one-base-per-tile path");
  constexpr int KS = D / 32;                 // k-steps of the QK^T product
  constexpr int DT = D / 16;                 // 16-row tiles of O^T
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int RPL = 64 / CPR;              // rows per direct-load instruction
  constexpr int NL = kBK / RPL / 4;          // direct-load instructions per wave per tile
  constexpr int ROWB = D * 2;                // bytes per K/V row in LDS
  constexpr int TILEB = kBK * ROWB;          // bytes per K (or V) tile
  // two buffers as distinct objects: with the tile loop unrolled by two, every LDS read of
  // one buffer is known not to alias the HBM->LDS loads in flight into the other, so no
  // wait on those loads is placed before the reads
  __shared__ __attribute__((aligned(1024))) char lds_a[2][TILEB];  // [K=0,V=1]
  __shared__ __attribute__((aligned(1024))) char lds_b[2][TILEB];

  // Work unit: (head group hg, sequence b, query tile t counted from the sequence end); it
  // reads ceil(Lk / 64) - t key tiles. blockIdx.x = hg runs fastest, so the workgroups of a
  // head group - dealt round-robin to the XCDs - stay on one XCD, where all its query tiles
  // share the K/V in L2. Plane z = blockIdx.z holds, for each sequence, the unit with
  // exactly nkt = gridDim.z - z key tiles, if the sequence has one: the dispatcher, which
  // hands workgroups out in index order, starts the longest units first. Within a plane the
  // sequences are rotated by z: consecutive workgroups go round-robin to the shader
  // engines of an XCD, and unrotated a sequence would meet the same engine in every plane,
  // leaving the engines that drew the long sequences with most of the work.
  auto unit = [&](const int hg, const int b, const int z) {
    const int G = num_heads / num_kv_heads;
    const int h0 = hg * GH, g = h0 / G;
    const int q_begin = cu_q[b];
    const int Lq = cu_q[b + 1] - q_begin;
    const int cap = bt_stride << bs_log2;
    int Lk = cu_k[b + 1] - cu_k[b];
    if constexpr (!PACKED) Lk = Lk > cap ? cap : Lk;
    const int t = (Lk + kBK - 1) / kBK - ((int)gridDim.z - z);
    if (t < 0) return;              // no unit of this length in this sequence
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
    const int32_t* bt = PACKED ? nullptr : block_tables + (int64_t)b * bt_stride;
    const int64_t k_row0 = PACKED ? cu_k[b] : 0;  // packed: the sequence's first key row
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

    // ---- direct HBM -> LDS tile loads -------------------------------------------------------
    // Instruction i of this wave fills LDS bytes [(wave*NL + i) * 1024, +1024) of a tile: rows
    // RPL * (wave*NL + i) + lane / CPR, slot lane % CPR. K slot s of row r holds chunk
    // s ^ (r % CPR); V slot s holds chunk 2 * ((s/2) ^ (r % (CPR/2))) + s % 2 (32-byte swizzle).
    int lrow[NL];
  #pragma unroll
    for (int i = 0; i < NL; ++i) lrow[i] = RPL * (wave * NL + i) + lane / CPR;
    const int slot = lane % CPR;
    int kchunk[NL], vchunk[NL];
  #pragma unroll
    for (int i = 0; i < NL; ++i) {
      kchunk[i] = slot ^ (lrow[i] % CPR);
      vchunk[i] = 2 * ((slot >> 1) ^ (lrow[i] % (CPR / 2))) + (slot & 1);
    }
    // BIG_BLOCKS: a tile's rows need one block id, and their addresses are that block's
    // base plus a per-lane constant. Otherwise every row looks its block up.
    int lane_off_k[NL], lane_off_v[NL];  // elements from the tile's first row
  #pragma unroll
    for (int i = 0; i < NL; ++i) {
      lane_off_k[i] = lrow[i] * (int)k_stride + g * D + 8 * kchunk[i];
      lane_off_v[i] = lrow[i] * (int)v_stride + g * D + 8 * vchunk[i];
    }
    int nblk[NL];  // block ids of this lane's rows for a tile two steps ahead
    // BIG_BLOCKS: lane l holds table column wbase + l (a vector load, so no scalar load is
    // in flight in the tile loop to force full lgkmcnt waits on the LDS reads)
    int win = -1, wbase = 0;
    const int ncols = (Lk + bs_mask) >> bs_log2;
    auto load_window = [&](int base) {
      wbase = base;
      const int c = base + lane;
      win = c < ncols ? bt[c] : -1;
    };
    auto fetch_blocks = [&](int kt) {
      if constexpr (PACKED) return;
      if constexpr (BIG_BLOCKS) {  // the tile's table column (nblk[1..] unused)
        if (kt < n_kt) {
          const int c = (kt * kBK) >> bs_log2;
          if (c - wbase >= 64) load_window(c);
          nblk[0] = c;
        } else {
          nblk[0] = -1;
        }
        return;
      }
  #pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int j = kt * kBK + lrow[i];
        nblk[i] = (kt < n_kt && j < Lk) ? bt[j >> bs_log2] : -1;
      }
    };
    auto issue_tile = [&](int kt, char (*dst)[TILEB], const int* blk) {
      if constexpr (BIG_BLOCKS) {
        bool blk_ok = true;
        int64_t base_k, base_v;
        if constexpr (PACKED) {
          base_k = (k_row0 + kt * kBK) * k_stride;
          base_v = (k_row0 + kt * kBK) * v_stride;
        } else {
          const int c0 = __builtin_amdgcn_readfirstlane(blk[0]);
          const int b0 = c0 >= 0 ? __builtin_amdgcn_readlane(win, c0 - wbase) : -1;
          blk_ok = (unsigned)b0 < (unsigned)num_blocks;
          base_k = blk_ok ? ((int64_t)b0 << bs_log2 | ((kt * kBK) & bs_mask)) * row_elems : 0;
          base_v = base_k;
        }
        const __bf16* kb = k_cache + base_k;
        const __bf16* vb = v_cache + base_v;
        if (blk_ok && (kt + 1) * kBK <= Lk) {  // a full tile of real keys: loads only
  #pragma unroll
          for (int i = 0; i < NL; ++i) {
            load_lds16_buf(kb, 2 * lane_off_k[i], &dst[0][(wave * NL + i) * 1024]);
            load_lds16_buf(vb, 2 * lane_off_v[i], &dst[1][(wave * NL + i) * 1024]);
          }
          return;
        }
  #pragma unroll
        for (int i = 0; i < NL; ++i) {  // the last tile of the keys, or a bad block id
          const int j = kt * kBK + lrow[i];
          char* kdst = &dst[0][(wave * NL + i) * 1024];
          char* vdst = &dst[1][(wave * NL + i) * 1024];
          if (blk_ok && j < Lk) {
            load_lds16_buf(kb, 2 * lane_off_k[i], kdst);
            load_lds16_buf(vb, 2 * lane_off_v[i], vdst);
          } else {
            // past the sequence: zeros; a bad block id: NaN (poisons only this sequence's rows)
            const u32x4_t fill = j < Lk ? Elem<__bf16>::nan_chunk() : u32x4_t{0u, 0u, 0u, 0u};
            store16(kdst + 16 * lane, fill);
            store16(vdst + 16 * lane, fill);
          }
        }
        return;
      }
      bool ok[NL];
      bool all_ok = true;
  #pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int j = kt * kBK + lrow[i];
        ok[i] = j < Lk && (unsigned)blk[i] < (unsigned)num_blocks;
        all_ok &= ok[i];
      }
      if (__all(all_ok)) {  // every row of the tile is a real key: loads only, no branches
  #pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int j = kt * kBK + lrow[i];
          const int64_t rowoff =
              (int64_t)((blk[i] << bs_log2) + (j & bs_mask)) * row_elems + (int64_t)g * D;
          load_lds16(k_cache + rowoff + 8 * kchunk[i], &dst[0][(wave * NL + i) * 1024]);
          load_lds16(v_cache + rowoff + 8 * vchunk[i], &dst[1][(wave * NL + i) * 1024]);
        }
        return;
      }
  #pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int j = kt * kBK + lrow[i];
        char* kdst = &dst[0][(wave * NL + i) * 1024];
        char* vdst = &dst[1][(wave * NL + i) * 1024];
        if (ok[i]) {
          const int64_t rowoff =
              (int64_t)((blk[i] << bs_log2) + (j & bs_mask)) * row_elems + (int64_t)g * D;
          load_lds16(k_cache + rowoff + 8 * kchunk[i], kdst);
          load_lds16(v_cache + rowoff + 8 * vchunk[i], vdst);
        } else {
          // past the sequence: zeros; a bad block id: NaN (poisons only this sequence's rows)
          const u32x4_t fill = j < Lk ? Elem<__bf16>::nan_chunk() : u32x4_t{0u, 0u, 0u, 0u};
          store16(kdst + 16 * lane, fill);
          store16(vdst + 16 * lane, fill);
        }
      }
    };

    f32x4_t oacc[DT][GH];
  #pragma unroll
    for (int i = 0; i < DT; ++i)
  #pragma unroll
      for (int nt = 0; nt < GH; ++nt) oacc[i][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // l_acc[nt]: the softmax denominators, accumulated by the PV MFMA with an all-ones A
    // operand (every lane ends with its column's sum over the keys of the probabilities it
    // fed to the PV product, bf16-rounded like them)
    float m_run[GH];
    f32x4_t l_acc[GH];
  #pragma unroll
    for (int nt = 0; nt < GH; ++nt) {
      m_run[nt] = -INFINITY;
      l_acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    int cblk[NL];
    if (n_kt > 0) {
      if constexpr (BIG_BLOCKS && !PACKED) load_window(0);
      fetch_blocks(0);
  #pragma unroll
      for (int i = 0; i < NL; ++i) cblk[i] = nblk[i];
      wait_vmem();
      issue_tile(0, lds_a, cblk);
      fetch_blocks(1);
    }
    auto tile_step = [&](int kt, char (*cur)[TILEB], char (*nxt)[TILEB]) {
      wait_vmem();          // this wave's part of tile kt (and the block ids of tile kt+1)
      __syncthreads();      // every wave's part; every wave is done with the other buffer
      if (kt + 1 < n_kt) {
  #pragma unroll
        for (int i = 0; i < NL; ++i) cblk[i] = nblk[i];
        issue_tile(kt + 1, nxt, cblk);
        fetch_blocks(kt + 2);
      }
      const char* Kt = cur[0];
      const char* Vt = cur[1];

      // S^T = K Q^T : sacc[mt][nt][r] = score of key kt*64 + 16 mt + 4 quad + r, column col
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
          for (int nt = 0; nt < GH; ++nt) sacc[mt][nt] = mfma16(ka[s & 1][mt], qb[nt][s], sacc[mt][nt]);
        }
      }
      // issue order: the 4 K reads of k-step 0, then each K read of step s+1 after the two
      // MFMAs of one 16-key block of step s, then the last step's MFMAs (without it the
      // compiler bunches the reads and waits for each pair right before its MFMAs)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  #pragma unroll
      for (int s = 0; s + 1 < KS; ++s)
  #pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          __builtin_amdgcn_sched_group_barrier(0x008, GH, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * GH, 0);

      // online softmax of the tile; the causal mask only on tiles that cross this wave's
      // diagonal. The reference max of a column (m_run) moves only when a tile's max exceeds
      // it by more than kSlack in log2 units (or was -inf): probabilities stay <= 2^kSlack,
      // O and l share the reference, and most tiles skip rescaling O altogether.
      bf16x8_t pb[2][GH];
      float mxs[GH];
      auto softmax = [&](auto masked) {
        constexpr bool kMask = decltype(masked)::value;
        bool need = false;
  #pragma unroll
        for (int nt = 0; nt < GH; ++nt) {
          float mx = -INFINITY;
  #pragma unroll
          for (int mt = 0; mt < 4; ++mt)
  #pragma unroll
            for (int r = 0; r < 4; ++r) {
              if constexpr (kMask) {
                const int j = kt * kBK + 16 * mt + 4 * quad + r;
                if (j > pos) sacc[mt][nt][r] = -INFINITY;
              }
              mx = fmaxf(mx, sacc[mt][nt][r]);
            }
          mxs[nt] = rows_max(mx);
          need |= (mxs[nt] - m_run[nt]) * scale_log2e > kSlack || (m_run[nt] == -INFINITY && mxs[nt] != -INFINITY);
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
      };
      if (kt * kBK + kBK - 1 > wave_min_pos)
        softmax(std::true_type{});
      else
        softmax(std::false_type{});

      // Probabilities 2^(s scale log2e - m) of the lane's keys, rounded to bf16 in the PV
      // operand layout. Those of the second 32 keys (ks = 1) are computed in pieces between
      // the MFMAs of the first 32 keys' PV product, which do not depend on them, so the
      // wavefront's own matrix and vector work overlap.
      float mcs[GH];
      float pv[GH][4][4];
  #pragma unroll
      for (int nt = 0; nt < GH; ++nt)
        mcs[nt] = (m_run[nt] == -INFINITY ? 0.f : m_run[nt]) * scale_log2e;
      auto prob = [&](int nt, int mt, int r) {
        pv[nt][mt][r] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][nt][r], scale_log2e, -mcs[nt]));
      };
      auto pack = [&](int ks) {
  #pragma unroll
        for (int nt = 0; nt < GH; ++nt) {
          u32x4_t w;
          w.x = pack_bf16x2(pv[nt][2 * ks][0], pv[nt][2 * ks][1]);
          w.y = pack_bf16x2(pv[nt][2 * ks][2], pv[nt][2 * ks][3]);
          w.z = pack_bf16x2(pv[nt][2 * ks + 1][0], pv[nt][2 * ks + 1][1]);
          w.w = pack_bf16x2(pv[nt][2 * ks + 1][2], pv[nt][2 * ks + 1][3]);
          pb[ks][nt] = __builtin_bit_cast(bf16x8_t, w);
        }
      };
  #pragma unroll
      for (int nt = 0; nt < GH; ++nt)
  #pragma unroll
        for (int mt = 0; mt < 2; ++mt)
  #pragma unroll
          for (int r = 0; r < 4; ++r) prob(nt, mt, r);
      pack(0);
      constexpr int kLate = GH * 2 * 4;             // probabilities of the second 32 keys
      constexpr int kPerStep = (kLate + DT - 1) / DT;  // computed after each of the DT steps

      // O^T += V^T P^T ; lane (row d = 16 i + col, group quad) reads keys 32 ks + 4 quad + 0..3
      // and 32 ks + 16 + 4 quad + 0..3 with two transposing reads. Source lane L of a group
      // points at key k0 + L / 4, dims 16 i + 4 (L % 4) .. + 3.
  #pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 1) pack(1);
  #pragma unroll
        for (int i = 0; i < DT; ++i) {
          s16x4_t part[2];
  #pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int r = 32 * ks + 16 * hf + 4 * quad + (col >> 2);
            const int c2 = i ^ (r % (CPR / 2));  // 32-byte chunk i, swizzled
            const char* src = Vt + r * ROWB + 32 * c2 + 8 * (col & 3);
            part[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)src);
          }
          u32x4_t w;
          w.x = __builtin_bit_cast(u32x2_t, part[0]).x;
          w.y = __builtin_bit_cast(u32x2_t, part[0]).y;
          w.z = __builtin_bit_cast(u32x2_t, part[1]).x;
          w.w = __builtin_bit_cast(u32x2_t, part[1]).y;
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, w);
  #pragma unroll
          for (int nt = 0; nt < GH; ++nt) oacc[i][nt] = mfma16(av, pb[ks][nt], oacc[i][nt]);
          if (ks == 0) {
  #pragma unroll
            for (int e = i * kPerStep; e < (i + 1) * kPerStep && e < kLate; ++e)
              prob(e / 8, 2 + (e / 4) % 2, e % 4);
          }
        }
      }
      const bf16x8_t ones = __builtin_bit_cast(
          bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  #pragma unroll
      for (int ks = 0; ks < 2; ++ks)
  #pragma unroll
        for (int nt = 0; nt < GH; ++nt) l_acc[nt] = mfma16(ones, pb[ks][nt], l_acc[nt]);
    };
    for (int kt = 0; kt < n_kt; kt += 2) {
      tile_step(kt, lds_a, lds_b);
      if (kt + 1 < n_kt) tile_step(kt + 1, lds_b, lds_a);
    }

    // normalise and store: lane holds dims 16 i + 4 quad + r of its query column
  #pragma unroll
    for (int nt = 0; nt < GH; ++nt) {
      const float inv = 1.f / l_acc[nt][0];
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
  };
  const int B = gridDim.y, z = blockIdx.z;
  int b = blockIdx.y + z % B;
  if (b >= B) b -= B;
  unit(blockIdx.x, b, z);
}

template <int D, int GH, bool BIG_BLOCKS, bool PACKED = false>
static int run_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int bs_log2 = PACKED ? 0 : __builtin_ctz((unsigned)a.block_size);
  const int64_t row = (int64_t)a.num_kv_heads * D;
  dim3 grid(a.num_heads / GH, a.num_seqs, a.key_tiles);
  hipLaunchKernelGGL((prefill_kernel<D, GH, BIG_BLOCKS, PACKED>), grid, dim3(256), 0, stream,
                     (__bf16*)a.out, (const __bf16*)a.q, (const __bf16*)a.k_cache,
                     (const __bf16*)a.v_cache, a.num_blocks, a.block_tables,
                     a.max_blocks_per_seq, a.cu_seqlens_q, a.cu_seqlens_k, a.num_heads,
                     a.num_kv_heads, bs_log2, a.scale * kLog2e, PACKED ? a.k_stride : row,
                     PACKED ? a.v_stride : row);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

template <int D, int GH>
static int run_prefill_bs(const PrefillArgs& a, hipStream_t stream) {
  if (a.packed) return run_prefill<D, GH, true, true>(a, stream);
  return a.block_size >= kBK ? run_prefill<D, GH, true>(a, stream) : run_prefill<D, GH, false>(a, stream);
}

int launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.key_tiles == 0) return 0;
  const int G = a.num_heads / a.num_kv_heads;
  const bool pair = (G % 2) == 0;
  if (a.head_dim == 128) return pair ? run_prefill_bs<128, 2>(a, stream) : run_prefill_bs<128, 1>(a, stream);
  if (a.head_dim == 64) return pair ? run_prefill_bs<64, 2>(a, stream) : run_prefill_bs<64, 1>(a, stream);
  return -2;
}

}  // namespace pkv
