// Paged decode attention with a split-K softmax, for gfx950.
//
// The operation is the decode branch of Attention.forward in "vLLM 学习笔记 02：nano-vllm
// 源码逐段精读": one query per sequence attends every cached key of the sequence (context
// length = len(seq), newest token included), K/V gathered through the block table.
//
// Work split (stream-K over the keys). Lay the work out as one line of key rows: for every
// sequence b in order and every kv head g, a segment of n_b = context_lens[b] keys. Every
// wavefront of the grid takes an equal, contiguous share S of that line (S is computed on
// the device from context_lens, never below `min_keys`), so each wavefront moves the same
// number of K/V bytes however the context lengths are spread. A share can start or end
// inside a segment and can cover several short segments; the part of a segment inside one
// share is a piece. A piece reads the K and V rows of its keys for head g only and serves
// all G query heads of the group, so each K/V byte leaves HBM once.
//
// Inside a wavefront a row of one head (D elements) is spread over LPR lanes, 16 bytes per
// lane, so one load instruction covers RPI rows; a chunk is NI such instructions (CH keys).
// The wavefront walks its share chunk by chunk with a two-deep register pipeline: the K and
// V loads of the next chunk are issued before the current chunk is computed, across piece
// boundaries too. Per chunk, the G dot products of each row (v_dot2_f32_bf16 on packed bf16,
// or fp32 FMAs) are summed over the row's lanes with DPP, and every row group (the lanes
// sharing one row slot) updates its own online-softmax state in log2 units:
//   m' = max(m, chunk max);  l, o scaled by 2^(m - m');  l += 2^(s - m');  o += 2^(s - m') v.
// At the end of a piece the row groups are merged with shuffles. A piece that is a whole
// segment writes the normalised output row; otherwise it writes (m, l, o) per query head
// into its slot, and decode_combine_kernel merges the slots of each (sequence, head):
//   M = max_p m_p, L = sum_p 2^(m_p - M) l_p, out = sum_p 2^(m_p - M) o_p / L.
// Keys past the context length are never loaded, so block-table padding and the unused
// (possibly NaN) slots of a sequence's last block are not touched. When the caller passes
// kv_stream_from (NT), sequence b's rows of table columns >= kv_stream_from[b] are read with
// non-temporal loads: the caller knows from its block manager that no other sequence of the
// call reads those blocks (prefix caching shares only leading blocks of a table), so keeping
// their rows in the caches would only displace lines that are read again - the shared
// leading blocks among them. The arithmetic is the same either way.
//
// Fused store (the store_kvcache that precedes decode attention in the engine's
// Attention.forward): the stream kernel takes n_b - 1 keys of each sequence from the cache
// and always writes partials; the combine kernel adds the newest token as one more piece,
// (m, l, o) = (scale <q, k_new>, 1, v_new) straight from the step's key/value rows, and its
// first wavefront of each kv head copies those rows into their slots. No kernel of the call
// reads the newest token's slot, so the copy needs no ordering against the attention.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "prefix_unit.hpp"

namespace pkv {

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ int clamp_ctx(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }

// The shared blocks' work units as extra workgroups behind the stream shares (UNITS).
struct PrefixUnits {
  const int32_t* g_ptr;
  const int32_t* g_members;
  const int32_t* g_col;
  float* pfx_o;
  float* pfx_ml;
  int32_t num_heads;
  int32_t n_hg;        // head groups per kv row (q heads / the unit's heads)
  int32_t num_groups;
  int32_t n_stream;    // workgroups 0 .. n_stream - 1 own the stream shares
};

// One chunk of a wavefront's share: keys [k, k + cnt) of segment (b, g).
struct Chunk {
  int x;          // position of the chunk's first key on the line
  int b, g, k, cnt;
  int seg_start;  // line position of key 0 of the segment
  int n;          // segment length (context length of b)
  bool piece_start, piece_end;
};

// PFX: kv_stream_from[b] is the count of sequence b's leading table columns shared with
// other sequences of the call, whose keys decode_prefix_unit takes: the line holds only the
// keys past them, all read non-temporally, and every segment leaves partials for the
// combine.
// UNITS (with PFX): one grid for the whole prefix-mode pass. Workgroups below pu.n_stream
// are the stream shares; the rest are decode_prefix_unit work units, head group fastest.
// The dispatcher starts workgroups in index order, so the units take the slots that the
// first shares to finish leave free while the last shares still stream. Batches of 512
// sequences, half sharing 2-8 leading blocks of 256 keys, went from 281-287 us per call
// with the units as a second kernel after this one to 271.5-276.3 us (flushed cache, same
// process, two parts), bitwise the same output; the second kernel on a forked stream,
// joined by events, took 287-291 us. The units need the two-wavefronts-per-SIMD register
// bound (256 VGPRs), which spills the stream shares of 8 q heads per kv head, and their
// 64 KB of LDS tiles (D = 128) next to the stream shares' per-sequence table must leave
// room for two workgroups per CU; calls outside either limit launch the units as their own
// kernel.
template <typename T, int D, int G, int NI, int HPW, bool NT, bool PFX = false,
          bool UNITS = false>
__global__ __launch_bounds__(256, UNITS ? 2 : 1) void decode_stream_kernel(
    T* __restrict__ out, const T* __restrict__ q, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, int32_t num_blocks, const int32_t* __restrict__ block_tables,
    int32_t bt_stride, const int32_t* __restrict__ context_lens, int32_t num_seqs,
    int32_t num_kv_heads, int32_t bs_log2, float scale_log2e, int32_t min_keys,
    int32_t max_pieces, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    int32_t* __restrict__ ws_meta, int32_t skip_last,
    const int32_t* __restrict__ kv_stream_from, PrefixUnits pu) {
  if constexpr (UNITS) {
    static_assert(PFX && Elem<T>::kBytes == 2, "the shared-block units are bf16 MFMA");
    if ((int)blockIdx.x >= pu.n_stream) {
      const int u = (int)blockIdx.x - pu.n_stream;
      const int hg = u % pu.n_hg, rest = u / pu.n_hg;
      decode_prefix_unit<D, (G % 2 == 0 ? 2 : 1)>(
          hg, rest % pu.num_groups, rest / pu.num_groups, (const __bf16*)q,
          (const __bf16*)k_cache, (const __bf16*)v_cache, num_blocks, block_tables, bt_stride,
          pu.g_ptr, pu.g_members, pu.g_col, pu.num_heads, num_kv_heads, bs_log2, scale_log2e,
          pu.pfx_o, pu.pfx_ml);
      return;
    }
  }
  using E = Elem<T>;
  constexpr bool kBF16 = E::kBytes == 2;
  constexpr int EPL = E::kPerChunk;  // elements per 16-byte lane chunk
  constexpr int LPR = D / EPL;       // lanes per row
  // HPW == 0: each wavefront owns a share of the (sequence, kv head) line and one head per
  // chunk. HPW > 0: each workgroup owns a share of the (sequence) line and its wavefront w
  // serves kv heads w*HPW .. w*HPW+HPW-1, so the group reads whole token rows together.
  constexpr int RSTRIDE = (HPW > 0 ? HPW : 1) * LPR;  // lanes between rows of one instruction
  constexpr int RPI = 64 / RSTRIDE;  // rows (keys) per load instruction
  constexpr int CH = RPI * NI;       // keys per chunk
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row must tile a wavefront");

  extern __shared__ int32_t s_cum[];  // [num_seqs + 1]: prefix sums of the context lengths

  const int cap = bt_stride << bs_log2;
  // Calls of more than 64 sequences (and prefix mode): every thread first loads lengths, up
  // to 4 per thread in one batch of loads, into s_cum[b + 1], and wave 0 scans them from
  // there - one round trip per 1024 sequences instead of one per 64, each cold after an idle
  // cache (batch 512 with shared prefixes: 263.3-266.0 -> 259.1-260.6 us per call).
  const bool staged = PFX || num_seqs > 64;
  if (staged) {
    for (int b0 = 0; b0 < num_seqs; b0 += 1024) {
      int n[4], f[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = b0 + 256 * u + (int)threadIdx.x;
        n[u] = b < num_seqs ? context_lens[b] : 0;
        f[u] = 0;
        if constexpr (PFX) f[u] = b < num_seqs ? kv_stream_from[b] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = b0 + 256 * u + (int)threadIdx.x;
        int v = clamp_ctx(n[u], cap);
        v -= skip_last & (v > 0);  // the newest token comes from the step's rows
        if constexpr (PFX) v = max(0, v - (f[u] << bs_log2));
        if (b < num_seqs) s_cum[b + 1] = v;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x < 64) {
    int carry = 0;
    for (int base = 0; base < num_seqs; base += 64) {
      const int b = base + threadIdx.x;
      int v = 0;
      if (staged) {
        v = b < num_seqs ? s_cum[b + 1] : 0;
      } else {
        v = b < num_seqs ? clamp_ctx(context_lens[b], cap) : 0;
        v -= skip_last & (v > 0);
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off);
        if ((int)threadIdx.x >= off) v += t;
      }
      if (b < num_seqs) s_cum[b + 1] = carry + v;
      carry += __shfl(v, 63);
    }
    if (threadIdx.x == 0) s_cum[0] = 0;
  }
  __syncthreads();

  const int Hkv = num_kv_heads;
  const int Hq = Hkv * G;
  const int mult = HPW > 0 ? 1 : Hkv;  // line positions per key of a sequence
  const int total = mult * s_cum[num_seqs];
  const int n_owner_blocks = UNITS ? pu.n_stream : (int)gridDim.x;
  const int n_waves = HPW > 0 ? n_owner_blocks : n_owner_blocks * 4;  // share owners
  int S = (total + n_waves - 1) / n_waves;
  S = S < min_keys ? min_keys : S;
  if (blockIdx.x == 0) {  // publish the split for the combine kernel
    for (int i = threadIdx.x; i <= num_seqs; i += 256) ws_meta[1 + i] = s_cum[i];
    if (threadIdx.x == 0) ws_meta[0] = S;
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w = HPW > 0 ? blockIdx.x : blockIdx.x * 4 + wave;  // share owner
  const int64_t xb = (int64_t)w * S;
  if (xb >= total) return;
  const int x_begin = (int)xb;
  const int x_end = (int)min((int64_t)total, xb + S);
  const int sub = lane % LPR, rsub = lane / RSTRIDE;
  const int g_lane = HPW > 0 ? wave * HPW + (lane / LPR) % HPW : 0;  // this lane's kv head
  const int64_t row_elems = (int64_t)Hkv * D;
  const int bs_mask = (1 << bs_log2) - 1;

  auto locate = [&](int x, Chunk& c) {
    int lo = 0, hi = num_seqs - 1;  // last b whose segments start at or before x
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mult * s_cum[mid] <= x) lo = mid; else hi = mid - 1;
    }
    c.b = lo;
    c.n = s_cum[lo + 1] - s_cum[lo];
    const int off = x - mult * s_cum[lo];
    c.g = HPW > 0 ? g_lane : off / c.n;
    c.k = HPW > 0 ? off : off - c.g * c.n;
    c.seg_start = x - c.k;
  };
  auto finish_desc = [&](Chunk& c, bool starts_piece) {
    const int seg_end = c.seg_start + c.n;
    c.cnt = min(CH, min(seg_end, x_end) - c.x);
    c.piece_start = starts_piece;
    c.piece_end = (c.x + c.cnt == seg_end) || (c.x + c.cnt == x_end);
  };
  auto next_of = [&](const Chunk& c, Chunk& nx) {
    nx.x = c.x + c.cnt;
    if (!c.piece_end) {  // same segment
      nx.b = c.b; nx.g = c.g; nx.n = c.n; nx.seg_start = c.seg_start; nx.k = c.k + c.cnt;
      finish_desc(nx, false);
    } else {
      locate(nx.x, nx);
      finish_desc(nx, true);
    }
  };
  // A window of 64 consecutive block-table entries of one sequence, one per lane; every kv
  // head of the sequence uses the same table, so the window is reloaded only when the
  // sequence changes or a chunk runs past it.
  int bt_b = -1, bt_base = 0, bt_reg = -1;
  int stream_from = INT32_MAX;  // first table column of sequence bt_b read non-temporally
  int pfx_b = -1, pfx_keys = 0;  // PFX: the shared leading keys of sequence pfx_b
  auto issue = [&](const Chunk& c, u32x4_t* kr, u32x4_t* vr) {
    if constexpr (PFX) {
      if (c.b != pfx_b) {
        pfx_b = c.b;
        pfx_keys = kv_stream_from[c.b] << bs_log2;
      }
    }
    const int k0 = PFX ? c.k + pfx_keys : c.k;  // the chunk's first key in the sequence
    const int first = k0 >> bs_log2, last = (k0 + c.cnt - 1) >> bs_log2;
    if (c.b != bt_b || first < bt_base || last >= bt_base + 64) {
      if constexpr (NT) {
        if (c.b != bt_b) stream_from = kv_stream_from[c.b];
      }
      bt_b = c.b;
      bt_base = first;
      bt_reg = bt_base + lane < bt_stride ? block_tables[(int64_t)c.b * bt_stride + bt_base + lane] : -1;
    }
    const int64_t head_off = (int64_t)c.g * D + sub * EPL;
    // a chunk inside one block (the usual case for blocks of >= 32 keys) reads its block id
    // once from the window with a scalar lane read; otherwise each row shuffles its own
    const bool one_block = first == last;
    const int blk0 = __builtin_amdgcn_readlane(bt_reg, min(first - bt_base, 63));
    // the chunk's loads as one straight batch per load kind (the choice is wave-uniform)
    auto loads = [&](auto streamed) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = i * RPI + rsub;
        const int j = k0 + r;
        const int blk = one_block ? blk0 : __shfl(bt_reg, min((j >> bs_log2) - bt_base, 63));
        kr[i] = u32x4_t{0u, 0u, 0u, 0u};
        vr[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (r < c.cnt) {
          if ((unsigned)blk < (unsigned)num_blocks) {
            const int64_t off = (((int64_t)blk << bs_log2) + (j & bs_mask)) * row_elems + head_off;
            if constexpr (decltype(streamed)::value) {
              kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(k_cache + off));
              vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(v_cache + off));
            } else {
              kr[i] = load16(k_cache + off);
              vr[i] = load16(v_cache + off);
            }
          } else {
            kr[i] = E::nan_chunk();
            vr[i] = E::nan_chunk();
          }
        }
      }
    };
    if (NT && first >= stream_from)
      loads(std::true_type{});
    else
      loads(std::false_type{});
  };
  auto load_q = [&](const Chunk& c, u32x4_t* qw) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      qw[h] = load16(q + ((int64_t)c.b * Hq + c.g * G + h) * D + sub * EPL);
  };

  float m[G], l[G], o[G][EPL];
  auto reset = [&]() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
    }
  };

  auto compute = [&](const Chunk& c, const u32x4_t* kr, const u32x4_t* vr, const u32x4_t* qw) {
    float qf[G][EPL];
    if constexpr (!kBF16) {
#pragma unroll
      for (int h = 0; h < G; ++h) E::unpack(qw[h], qf[h]);
    }
    float s[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[EPL];
      if constexpr (!kBF16) E::unpack(kr[i], kf);
      const bool valid = i * RPI + rsub < c.cnt;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
        if constexpr (kBF16) {
          acc = dot2_bf16(kr[i].x, qw[h].x, acc);
          acc = dot2_bf16(kr[i].y, qw[h].y, acc);
          acc = dot2_bf16(kr[i].z, qw[h].z, acc);
          acc = dot2_bf16(kr[i].w, qw[h].w, acc);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc = fmaf(qf[h][e], kf[e], acc);
        }
        acc = group_sum<LPR>(acc) * scale_log2e;
        s[i][h] = valid ? acc : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mc = s[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) mc = fmaxf(mc, s[i][h]);
      const float m_new = fmaxf(m[h], mc);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[h] - m_use);
      m[h] = m_new;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) s[i][h] = __builtin_amdgcn_exp2f(s[i][h] - m_use);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[EPL];
      E::unpack(vr[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        l[h] += s[i][h];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(s[i][h], vf[e], o[h][e]);
      }
    }
  };

  auto finalize = [&](const Chunk& c, int piece_x0) {
    // merge the row groups (lanes with equal `sub`)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mall = m[h];
#pragma unroll
      for (int msk = RSTRIDE; msk < 64; msk <<= 1) mall = fmaxf(mall, __shfl_xor(mall, msk));
      const float muse = mall == -INFINITY ? 0.f : mall;
      const float sc = __builtin_amdgcn_exp2f(m[h] - muse);
      float lt = l[h] * sc;
#pragma unroll
      for (int msk = RSTRIDE; msk < 64; msk <<= 1) lt += __shfl_xor(lt, msk);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float v = o[h][e] * sc;
#pragma unroll
        for (int msk = RSTRIDE; msk < 64; msk <<= 1) v += __shfl_xor(v, msk);
        o[h][e] = v;
      }
      m[h] = mall;
      l[h] = lt;
    }
    if (rsub == 0) {
      const bool whole = !PFX && !skip_last && piece_x0 == c.seg_start &&
                         c.x + c.cnt == c.seg_start + c.n;
      if (whole) {
        T* dst0 = out + ((int64_t)c.b * Hq + c.g * G) * D + sub * EPL;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float inv = 1.f / l[h];
          T* dst = dst0 + h * D;
          if constexpr (kBF16) {
            u32x4_t wv;
            wv.x = pack_bf16x2(o[h][0] * inv, o[h][1] * inv);
            wv.y = pack_bf16x2(o[h][2] * inv, o[h][3] * inv);
            wv.z = pack_bf16x2(o[h][4] * inv, o[h][5] * inv);
            wv.w = pack_bf16x2(o[h][6] * inv, o[h][7] * inv);
            store16(dst, wv);
          } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) E::store(dst + e, o[h][e] * inv);
          }
        }
      } else {
        const int piece = w - c.seg_start / S;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const int64_t slot = ((int64_t)c.b * Hq + c.g * G + h) * max_pieces + piece;
          float* dst = ws_o + slot * D + sub * EPL;
#pragma unroll
          for (int e = 0; e < EPL; e += 4)
            store16(dst + e, u32x4_t{__float_as_uint(o[h][e]), __float_as_uint(o[h][e + 1]),
                                     __float_as_uint(o[h][e + 2]), __float_as_uint(o[h][e + 3])});
          if (sub == 0) {
            ws_ml[2 * slot] = m[h];
            ws_ml[2 * slot + 1] = l[h];
          }
        }
      }
    }
    reset();
  };

  // ---- the pipeline: two register buffers, next chunk issued before the current computes --
  u32x4_t kA[NI], vA[NI], kB[NI], vB[NI];
  u32x4_t qc[G], qn[G];
  Chunk cur, nxt;
  cur.x = x_begin;
  locate(x_begin, cur);
  finish_desc(cur, true);
  load_q(cur, qc);
  issue(cur, kA, vA);
  reset();
  int piece_x0 = x_begin;

  auto half_step = [&](u32x4_t* kc, u32x4_t* vc, u32x4_t* kn, u32x4_t* vn) -> bool {
    const bool has_next = cur.x + cur.cnt < x_end;
    if (has_next) {
      next_of(cur, nxt);
      if (nxt.piece_start) load_q(nxt, qn);
      issue(nxt, kn, vn);
    }
    compute(cur, kc, vc, qc);
    if (cur.piece_end) finalize(cur, piece_x0);
    if (!has_next) return false;
    if (nxt.piece_start) {
#pragma unroll
      for (int h = 0; h < G; ++h) qc[h] = qn[h];
      piece_x0 = nxt.x;
    }
    cur = nxt;
    return true;
  };
  // The SIMD issues from its oldest ready wavefront first, so the workgroups dispatched
  // first to a CU would stream ahead of the ones dispatched after them and the latter set
  // the kernel's end. Alternating every wavefront's priority from chunk to chunk keeps any
  // one of them from being favoured for long (measured: -1.5% at batch 64, -2% at 512).
  while (true) {
    __builtin_amdgcn_s_setprio(1);
    if (!half_step(kA, vA, kB, vB)) break;
    __builtin_amdgcn_s_setprio(0);
    if (!half_step(kB, vB, kA, vA)) break;
  }
}

// D / 64 elements of one row per lane, as raw bits (a copy) or as floats.
template <typename T, int DPL> struct LaneBits;
template <> struct LaneBits<__bf16, 1> { typedef uint16_t type; };
template <> struct LaneBits<__bf16, 2> { typedef uint32_t type; };
template <> struct LaneBits<float, 1> { typedef uint32_t type; };
template <> struct LaneBits<float, 2> { typedef u32x2_t type; };
template <typename T, int DPL>
__device__ __forceinline__ void bits_to_float(const typename LaneBits<T, DPL>::type& w, float* f) {
  if constexpr (Elem<T>::kBytes == 2) {
    if constexpr (DPL == 2) { f[0] = bf16_lo(w); f[1] = bf16_hi(w); }
    else f[0] = __uint_as_float((uint32_t)w << 16);
  } else {
    if constexpr (DPL == 2) { f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y); }
    else f[0] = __uint_as_float(w);
  }
}

// Merges the partial slots of every (sequence, query head) whose segment was split: one
// wavefront per (sequence, head), four per workgroup (calls of many rows; few rows go to
// decode_combine_wide_kernel). The kernel is latency bound, so it takes two rounds of loads:
// first the split metadata together with the (m, l) of the first 64 slots (lane p holds slot
// p; the slots exist for every row, so they are read before the row's slot count is known),
// the o rows of the first kSpec slots and, for the fused store, q and the newest token's
// rows; then the o rows of the remaining slots, up to 16 at a time, D / 64 consecutive floats
// per lane (one coalesced row per load instruction). A row cut into at most kSpec pieces
// needs no second round. kSpec is 16 for calls of at most 128 sequences, whose rows are cut
// into more pieces (a share then covers a few hundred keys), and 4 for larger ones, where
// most rows have one or two pieces and 16 speculative rows per row would be mostly wasted
// (1 for larger ones in prefix mode, whose rows merge their shared pieces later anyway).
// PFX: besides the stream kernel's pieces, row (b, h) merges one piece per shared leading
// table column of sequence b (pp.cols[b] of them), left by the decode_prefix_unit work units.
template <typename T, int D, int kSpec, bool PFX = false>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    T* __restrict__ out, const int32_t* __restrict__ context_lens, int32_t cap,
    int32_t num_rows, int32_t Hq, int32_t Hkv, int32_t max_pieces,
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ ws_meta, int32_t per_seq_line, NewTokens nt,
    PrefixParts pp) {
  constexpr int DPL = D / 64;  // floats per lane
  constexpr int OB = 16;       // o rows per load batch
  static_assert(DPL == 1 || DPL == 2, "head_dim 64 or 128");
  typedef typename LaneBits<T, DPL>::type Bits;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // b * Hq + h
  if (row >= num_rows) return;
  const int b = row / Hq, h = row - b * Hq;
  const int g = h / (Hq / Hkv);
  const int64_t base = (int64_t)row * max_pieces;
  const bool fused = nt.key != nullptr;
  // first batch of loads
  const int n_raw = context_lens[b];
  const int S = ws_meta[0];
  const int cum = ws_meta[1 + b];
  float mp = -INFINITY, lp = 0.f;
  if (lane < max_pieces) {
    mp = ws_ml[2 * (base + lane)];
    lp = ws_ml[2 * (base + lane) + 1];
  }
  float ov0[kSpec][DPL];
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    const float* src = ws_o + (base + min(u, max_pieces - 1)) * D + lane * DPL;
    if constexpr (DPL == 2) {
      const float2 v = *reinterpret_cast<const float2*>(src);
      ov0[u][0] = v.x;
      ov0[u][1] = v.y;
    } else {
      ov0[u][0] = *src;
    }
  }
  Bits qw{}, kw{}, vw{};
  int slot = -1;
  if (fused) {
    const int64_t col = (int64_t)g * D + lane * DPL;
    qw = *reinterpret_cast<const Bits*>(reinterpret_cast<const T*>(nt.q) + (int64_t)row * D + lane * DPL);
    kw = *reinterpret_cast<const Bits*>(reinterpret_cast<const T*>(nt.key) + b * nt.key_stride + col);
    vw = *reinterpret_cast<const Bits*>(reinterpret_cast<const T*>(nt.value) + b * nt.value_stride + col);
    slot = nt.slot_mapping[b];
  }
  const int n = clamp_ctx(n_raw, cap);
  int nc = fused ? n - (n > 0) : n;  // keys the stream kernel took from the cache
  int pc = 0;                        // PFX: shared leading columns, merged from pp
  if constexpr (PFX) {
    pc = pp.cols[b];
    nc = max(0, nc - (pc << pp.bs_log2));
  }
  T* dst = out + (int64_t)row * D + lane * DPL;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  float M = -INFINITY;
  float L = 0.f;
  if (nc > 0) {
    // start of the segment on the split line: one per (sequence, kv head), or one per sequence
    const int seg_start = per_seq_line ? cum : Hkv * cum + g * nc;
    const int np = (seg_start + nc - 1) / S - seg_start / S + 1;
    if (np == 1 && !fused && !PFX) return;  // written by the stream kernel
    for (int p0 = 0; p0 < np; p0 += 64) {
      const int cnt = min(64, np - p0);
      if (p0 > 0) {  // slots past the first 64 (segments cut into more than 64 pieces)
        mp = -INFINITY;
        lp = 0.f;
        if (lane < cnt) {
          mp = ws_ml[2 * (base + p0 + lane)];
          lp = ws_ml[2 * (base + p0 + lane) + 1];
        }
      } else if (lane >= cnt) {
        mp = -INFINITY;
        lp = 0.f;
      }
      const float Mn = fmaxf(M, group_max<64>(mp));
      const float rescale = __builtin_amdgcn_exp2f(M - Mn);
      const float wp = lane < cnt ? __builtin_amdgcn_exp2f(mp - Mn) : 0.f;
      L = fmaf(L, rescale, group_sum<64>(wp * lp));
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] *= rescale;
      M = Mn;
      // further batches: the o rows not loaded yet
      for (int p = 0; p < cnt; p += OB) {
        float ov[OB][DPL];
#pragma unroll
        for (int u = 0; u < OB; ++u) {
          if (u < kSpec && p0 == 0 && p == 0) {
#pragma unroll
            for (int e = 0; e < DPL; ++e) ov[u][e] = ov0[u < kSpec ? u : 0][e];
            continue;
          }
          if (p + u >= cnt) continue;
          const float* src = ws_o + (base + p0 + p + u) * D + lane * DPL;
          if constexpr (DPL == 2) {
            const float2 v = *reinterpret_cast<const float2*>(src);
            ov[u][0] = v.x;
            ov[u][1] = v.y;
          } else {
            ov[u][0] = *src;
          }
        }
#pragma unroll
        for (int u = 0; u < OB; ++u) {
          if (p + u >= cnt) break;
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wp), p + u));
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, ov[u][e], acc[e]);
        }
      }
    }
  }
  if constexpr (PFX) {
    // the shared blocks' pieces: slot (row, column c) for c < pc
    const int64_t pbase = (int64_t)row * pp.stride;
    for (int p0 = 0; p0 < pc; p0 += 64) {
      const int cnt = min(64, pc - p0);
      float mq = -INFINITY, lq = 0.f;
      if (lane < cnt) {
        mq = pp.ml[2 * (pbase + p0 + lane)];
        lq = pp.ml[2 * (pbase + p0 + lane) + 1];
      }
      const float Mn = fmaxf(M, group_max<64>(mq));
      const float rescale = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      const float wq = lane < cnt ? __builtin_amdgcn_exp2f(mq - Mn) : 0.f;
      L = fmaf(L, rescale, group_sum<64>(wq * lq));
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] *= rescale;
      M = Mn;
      for (int p = 0; p < cnt; p += 8) {
        float ov[8][DPL];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (p + u >= cnt) break;
          const float* src = pp.o + (pbase + p0 + p + u) * D + lane * DPL;
#pragma unroll
          for (int e = 0; e < DPL; ++e) ov[u][e] = src[e];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (p + u >= cnt) break;
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), p + u));
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, ov[u][e], acc[e]);
        }
      }
    }
  }
  if (fused) {
    if (n > 0) {  // the newest token as one more piece: m = scale <q, k>, l = 1, o = v
      float qf[DPL], kf[DPL], vf[DPL];
      bits_to_float<T, DPL>(qw, qf);
      bits_to_float<T, DPL>(kw, kf);
      bits_to_float<T, DPL>(vw, vf);
      float sd = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) sd = fmaf(qf[e], kf[e], sd);
      const float ms = group_sum<64>(sd) * nt.scale_log2e;
      const float Mn = fmaxf(M, ms);
      const float rescale = __builtin_amdgcn_exp2f(M - Mn);
      const float wn = __builtin_amdgcn_exp2f(ms - Mn);
      L = fmaf(L, rescale, wn);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(acc[e], rescale, wn * vf[e]);
    }
    // one wavefront per kv head stores the step's K/V rows (bit for bit) into their slot
    if (h % (Hq / Hkv) == 0 && slot >= 0 && (int64_t)slot < nt.num_slots) {
      const int64_t off = (int64_t)slot * Hkv * D + (int64_t)g * D + lane * DPL;
      *reinterpret_cast<Bits*>(reinterpret_cast<T*>(nt.k_cache) + off) = kw;
      *reinterpret_cast<Bits*>(reinterpret_cast<T*>(nt.v_cache) + off) = vw;
    }
  }
  if (n == 0) L = 1.f;  // a sequence with context length 0 gets a zero row
  const float inv = 1.f / L;
  if constexpr (DPL == 2) {
    if constexpr (Elem<T>::kBytes == 2) {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      *reinterpret_cast<float2*>(dst) = float2{acc[0] * inv, acc[1] * inv};
    }
  } else {
    Elem<T>::store(dst, acc[0] * inv);
  }
}

// Merges the partial slots of one (sequence, query head) per workgroup, for calls of few rows
// (a small batch, where the merge's cost is its latency and the few workgroups of the
// one-wavefront-per-row form leave most of the chip idle): wavefront w takes slots w*16 ..
// w*16+15 of every 64, so one round of loads covers a row of up to 64 pieces; the four
// wavefronts' (m, l, o) are then merged through LDS by wavefront 0, which also adds the
// newest token (fused store) and writes the row.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_wide_kernel(
    T* __restrict__ out, const int32_t* __restrict__ context_lens, int32_t cap,
    int32_t num_rows, int32_t Hq, int32_t Hkv, int32_t max_pieces,
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ ws_meta, int32_t per_seq_line, NewTokens nt) {
  constexpr int DPL = D / 64;
  constexpr int SPW = 16;  // slots per wavefront per round
  static_assert(DPL == 1 || DPL == 2, "head_dim 64 or 128");
  typedef typename LaneBits<T, DPL>::type Bits;
  __shared__ float s_part[4][2 + 64 * DPL];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x;  // b * Hq + h
  if (row >= num_rows) return;
  const int b = row / Hq, h = row - b * Hq;
  const int g = h / (Hq / Hkv);
  const int64_t base = (int64_t)row * max_pieces;
  const bool fused = nt.key != nullptr;
  // first batch of loads: metadata, this wavefront's first 16 slots, and (wavefront 0) the
  // newest token
  const int n_raw = context_lens[b];
  const int S = ws_meta[0];
  const int cum = ws_meta[1 + b];
  auto load_slots = [&](int p0, float& mp, float& lp, float (*ov)[DPL]) {
    const int s0 = p0 + wave * SPW;
    mp = -INFINITY;
    lp = 0.f;
    if (lane < SPW && s0 + lane < max_pieces) {
      mp = ws_ml[2 * (base + s0 + lane)];
      lp = ws_ml[2 * (base + s0 + lane) + 1];
    }
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const float* src = ws_o + (base + min(s0 + u, max_pieces - 1)) * D + lane * DPL;
      if constexpr (DPL == 2) {
        const float2 v = *reinterpret_cast<const float2*>(src);
        ov[u][0] = v.x;
        ov[u][1] = v.y;
      } else {
        ov[u][0] = *src;
      }
    }
  };
  float mp, lp, ov[SPW][DPL];
  load_slots(0, mp, lp, ov);
  Bits qw{}, kw{}, vw{};
  int slot = -1;
  if (fused && wave == 0) {
    const int64_t col = (int64_t)g * D + lane * DPL;
    qw = *reinterpret_cast<const Bits*>(reinterpret_cast<const T*>(nt.q) + (int64_t)row * D + lane * DPL);
    kw = *reinterpret_cast<const Bits*>(reinterpret_cast<const T*>(nt.key) + b * nt.key_stride + col);
    vw = *reinterpret_cast<const Bits*>(reinterpret_cast<const T*>(nt.value) + b * nt.value_stride + col);
    slot = nt.slot_mapping[b];
  }
  const int n = clamp_ctx(n_raw, cap);
  const int nc = fused ? n - (n > 0) : n;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  float M = -INFINITY, L = 0.f;
  if (nc > 0) {
    const int seg_start = per_seq_line ? cum : Hkv * cum + g * nc;
    const int np = (seg_start + nc - 1) / S - seg_start / S + 1;
    if (np == 1 && !fused) return;  // written by the stream kernel (uniform over the group)
    for (int p0 = 0; p0 < np; p0 += 4 * SPW) {
      if (p0 > 0) load_slots(p0, mp, lp, ov);
      const int s0 = p0 + wave * SPW;
      const int cnt = max(0, min(SPW, np - s0));  // this wavefront's slots in the round
      if (lane >= cnt) {
        mp = -INFINITY;
        lp = 0.f;
      }
      if (cnt == 0) continue;
      const float Mn = fmaxf(M, group_max<64>(mp));
      const float rescale = __builtin_amdgcn_exp2f(M - Mn);
      const float wp = lane < cnt ? __builtin_amdgcn_exp2f(mp - Mn) : 0.f;
      L = fmaf(L, rescale, group_sum<64>(wp * lp));
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] *= rescale;
      M = Mn;
#pragma unroll
      for (int u = 0; u < SPW; ++u) {
        if (u >= cnt) break;
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wp), u));
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, ov[u][e], acc[e]);
      }
    }
  }
  // the four wavefronts' states, merged by wavefront 0
  if (lane == 0) {
    s_part[wave][0] = M;
    s_part[wave][1] = L;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) s_part[wave][2 + lane * DPL + e] = acc[e];
  __syncthreads();
  if (wave != 0) return;
  M = fmaxf(fmaxf(s_part[0][0], s_part[1][0]), fmaxf(s_part[2][0], s_part[3][0]));
  const float Mu = M == -INFINITY ? 0.f : M;
  L = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float sc = __builtin_amdgcn_exp2f(s_part[w][0] - Mu);
    L = fmaf(sc, s_part[w][1], L);
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = fmaf(sc, s_part[w][2 + lane * DPL + e], acc[e]);
  }
  if (fused) {
    if (n > 0) {  // the newest token as one more piece: m = scale <q, k>, l = 1, o = v
      float qf[DPL], kf[DPL], vf[DPL];
      bits_to_float<T, DPL>(qw, qf);
      bits_to_float<T, DPL>(kw, kf);
      bits_to_float<T, DPL>(vw, vf);
      float sd = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) sd = fmaf(qf[e], kf[e], sd);
      const float ms = group_sum<64>(sd) * nt.scale_log2e;
      const float Mn = fmaxf(M, ms);
      const float rescale = __builtin_amdgcn_exp2f(M - Mn);
      const float wn = __builtin_amdgcn_exp2f(ms - Mn);
      L = fmaf(L, rescale, wn);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(acc[e], rescale, wn * vf[e]);
    }
    // one wavefront per kv head stores the step's K/V rows (bit for bit) into their slot
    if (h % (Hq / Hkv) == 0 && slot >= 0 && (int64_t)slot < nt.num_slots) {
      const int64_t off = (int64_t)slot * Hkv * D + (int64_t)g * D + lane * DPL;
      *reinterpret_cast<Bits*>(reinterpret_cast<T*>(nt.k_cache) + off) = kw;
      *reinterpret_cast<Bits*>(reinterpret_cast<T*>(nt.v_cache) + off) = vw;
    }
  }
  if (n == 0) L = 1.f;  // a sequence with context length 0 gets a zero row
  const float inv = 1.f / L;
  T* dst = out + (int64_t)row * D + lane * DPL;
  if constexpr (DPL == 2) {
    if constexpr (Elem<T>::kBytes == 2) {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      *reinterpret_cast<float2*>(dst) = float2{acc[0] * inv, acc[1] * inv};
    }
  } else {
    Elem<T>::store(dst, acc[0] * inv);
  }
}

// Calls of at most this many (sequence, q head) rows merge with one workgroup per row
// (decode_combine_wide_kernel). Measured per layer of a recorded 28-layer decode step, 16 q
// heads: batch 1 17.7 -> 15.7 us with the wide merge (one wavefront per row before), batch 4
// 21.8 -> 19.4, batch 16 -2 us; batch 64 (1024 rows) +0.5 us, so many rows keep one
// wavefront per row.
constexpr int kCombineFewRows = 256;
// Larger calls of at most this many sequences load the o rows of 16 slots in the combine's
// first round (batch 64, ~9 pieces per row: 94.7 -> 94.2 us per call, four alternating runs).
constexpr int kCombineSpec16Seqs = 128;

template <typename T, int D, int G, int NI, int HPW>
static int run_decode(const DecodeArgs& a, hipStream_t stream) {
  const int bs_log2 = __builtin_ctz((unsigned)a.block_size);
  const float c = a.scale * kLog2e;
  const int64_t cap = (int64_t)a.max_blocks_per_seq * a.block_size;
  // share owners: workgroups (HPW > 0) or wavefronts, never more than min_keys keys apart
  const int64_t upper = (int64_t)a.num_seqs * cap * (HPW > 0 ? 1 : a.num_kv_heads);
  const int64_t per_block = HPW > 0 ? a.partition : 4LL * a.partition;
  int64_t blocks = (upper + per_block - 1) / per_block;
  if (blocks > a.max_workgroups) blocks = a.max_workgroups;
  if (blocks < 1) blocks = 1;
  const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int32_t);
  auto* stream_kernel = a.kv_stream_from ? decode_stream_kernel<T, D, G, NI, HPW, true>
                                         : decode_stream_kernel<T, D, G, NI, HPW, false>;
  constexpr bool kPrefixMode = Elem<T>::kBytes == 2;  // the shared-block pass is bf16 MFMA
  // the shared-block units ride in the stream grid when its register bound fits the stream
  // shares (not with 8 q heads per kv head), two workgroups per CU still fit in LDS with the
  // units' tiles (D = 128: up to 4095 sequences) and the 1-D grid holds them all
  bool units_in_grid = false;
  int64_t units = 0;  // the units' workgroups (some exit at once: groups below the largest)
  if constexpr (kPrefixMode && G <= 4) {
    if (a.prefix && a.pfx.num_groups > 0 && a.pfx.max_group_size > 0)
      units = (int64_t)(a.num_heads / (G % 2 == 0 ? 2 : 1)) * a.pfx.num_groups *
              ((a.pfx.max_group_size + 63) / 64);
    units_in_grid = a.prefix != 0 &&
                    2 * (kPrefixUnitLds<D> + lds) <= (size_t)kLdsPerCu &&
                    blocks + units <= 0x7FFFFFFF;
  }
  if constexpr (kPrefixMode) {
    if (a.prefix && !units_in_grid) stream_kernel = decode_stream_kernel<T, D, G, NI, HPW, true, true>;
  }
  if (!units_in_grid) {
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(256),
                       lds, stream, (T*)a.out, (const T*)a.q, (const T*)a.k_cache,
                       (const T*)a.v_cache, a.num_blocks, a.block_tables, a.max_blocks_per_seq,
                       a.context_lens, a.num_seqs, a.num_kv_heads, bs_log2, c, a.partition,
                       a.max_parts, a.ws_o, a.ws_ml, a.ws_meta, a.new_k != nullptr ? 1 : 0,
                       a.kv_stream_from, PrefixUnits{});
  }
  PrefixParts pp{};
  if constexpr (kPrefixMode) {
    if (a.prefix) {
      if (units_in_grid) {
        if constexpr (G <= 4) {
          constexpr int GH = G % 2 == 0 ? 2 : 1;
          PrefixUnits pu;
          pu.g_ptr = a.pfx.group_ptr;
          pu.g_members = a.pfx.group_members;
          pu.g_col = a.pfx.group_col;
          pu.pfx_o = a.pfx.pfx_o;
          pu.pfx_ml = a.pfx.pfx_ml;
          pu.num_heads = a.num_heads;
          pu.n_hg = a.num_heads / GH;
          pu.num_groups = a.pfx.num_groups;
          pu.n_stream = (int32_t)blocks;
          hipLaunchKernelGGL((decode_stream_kernel<T, D, G, NI, HPW, true, true, true>),
                             dim3((unsigned)(blocks + units)), dim3(256), lds, stream,
                             (T*)a.out, (const T*)a.q, (const T*)a.k_cache,
                             (const T*)a.v_cache, a.num_blocks, a.block_tables,
                             a.max_blocks_per_seq, a.context_lens, a.num_seqs, a.num_kv_heads,
                             bs_log2, c, a.partition, a.max_parts, a.ws_o, a.ws_ml, a.ws_meta,
                             a.new_k != nullptr ? 1 : 0, a.kv_stream_from, pu);
        }
        if (hipGetLastError() != hipSuccess) return -4;
      } else {
        if (hipGetLastError() != hipSuccess) return -4;
        const int rc = launch_decode_prefix(a.pfx, stream);
        if (rc != 0) return rc;
      }
      pp = PrefixParts{a.kv_stream_from, a.pfx.pfx_o, a.pfx.pfx_ml, a.max_blocks_per_seq, bs_log2};
    }
  }
  const int rows = a.num_seqs * a.num_heads;
  NewTokens nt;
  nt.q = a.q;
  nt.key = a.new_k;
  nt.key_stride = a.new_k_stride;
  nt.value = a.new_v;
  nt.value_stride = a.new_v_stride;
  nt.slot_mapping = a.slot_mapping;
  nt.k_cache = const_cast<void*>(a.k_cache);
  nt.v_cache = const_cast<void*>(a.v_cache);
  nt.num_slots = a.num_slots;
  nt.scale_log2e = c;
  const dim3 cgrid((unsigned)((rows + 3) / 4));
  if constexpr (kPrefixMode) {
    // the shared blocks' pieces merge in the one-wavefront-per-row form. Larger calls load
    // one o row in the first round, not four: every row then merges its shared pieces in
    // later rounds anyway, and the 3 extra rows per row were mostly unused reads (batch 512,
    // half the sequences sharing 2-8 blocks: 266.3-267.0 -> 265.0-266.9 us per call, four
    // alternating reps, bitwise the same output)
    if (a.prefix) {
      if (a.num_seqs <= kCombineSpec16Seqs)
        hipLaunchKernelGGL((decode_combine_kernel<T, D, 16, true>), cgrid, dim3(256), 0, stream,
                           (T*)a.out, a.context_lens, (int32_t)cap, rows, a.num_heads,
                           a.num_kv_heads, a.max_parts, a.ws_o, a.ws_ml, a.ws_meta,
                           HPW > 0 ? 1 : 0, nt, pp);
      else
        hipLaunchKernelGGL((decode_combine_kernel<T, D, 1, true>), cgrid, dim3(256), 0, stream,
                           (T*)a.out, a.context_lens, (int32_t)cap, rows, a.num_heads,
                           a.num_kv_heads, a.max_parts, a.ws_o, a.ws_ml, a.ws_meta,
                           HPW > 0 ? 1 : 0, nt, pp);
      return hipGetLastError() == hipSuccess ? 0 : -4;
    }
  }
  if (rows <= kCombineFewRows)
    hipLaunchKernelGGL((decode_combine_wide_kernel<T, D>), dim3((unsigned)rows), dim3(256), 0,
                       stream, (T*)a.out, a.context_lens, (int32_t)cap, rows, a.num_heads,
                       a.num_kv_heads, a.max_parts, a.ws_o, a.ws_ml, a.ws_meta, HPW > 0 ? 1 : 0,
                       nt);
  else if (a.num_seqs <= kCombineSpec16Seqs)
    hipLaunchKernelGGL((decode_combine_kernel<T, D, 16>), cgrid, dim3(256), 0, stream,
                       (T*)a.out, a.context_lens, (int32_t)cap, rows, a.num_heads,
                       a.num_kv_heads, a.max_parts, a.ws_o, a.ws_ml, a.ws_meta, HPW > 0 ? 1 : 0,
                       nt, pp);
  else
    hipLaunchKernelGGL((decode_combine_kernel<T, D, 4>), cgrid, dim3(256), 0, stream,
                       (T*)a.out, a.context_lens, (int32_t)cap, rows, a.num_heads,
                       a.num_kv_heads, a.max_parts, a.ws_o, a.ws_ml, a.ws_meta, HPW > 0 ? 1 : 0,
                       nt, pp);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Whole token rows per workgroup when the kv heads split evenly over its 4 wavefronts and
// one load instruction still covers whole rows; otherwise one head per wavefront share. A
// call too small to give every workgroup of the grid a full share also takes one head per
// wavefront: its shares then start four times as many key streams at once (measured, per
// layer of a recorded 28-layer step with 8 kv heads: batch 1 -2.0 us, batch 4 -1.9 us).
template <typename T, int D, int G, int NI>
static int run_decode_hpw(const DecodeArgs& a, hipStream_t s) {
  constexpr int LPR = D / Elem<T>::kPerChunk;
  const bool small = (int64_t)a.num_seqs * a.max_blocks_per_seq * a.block_size <
                     (int64_t)a.max_workgroups * a.partition;
  switch (a.num_kv_heads % 4 == 0 && !small ? a.num_kv_heads / 4 : 0) {
    case 1: return run_decode<T, D, G, NI, 1>(a, s);
    case 2:
      if constexpr (2 * LPR <= 64) return run_decode<T, D, G, NI, 2>(a, s);
      return run_decode<T, D, G, NI, 0>(a, s);
    case 4:
      if constexpr (4 * LPR <= 64) return run_decode<T, D, G, NI, 4>(a, s);
      return run_decode<T, D, G, NI, 0>(a, s);
    default: return run_decode<T, D, G, NI, 0>(a, s);
  }
}

template <typename T, int D>
static int dispatch_g(const DecodeArgs& a, hipStream_t s) {
  // A call that fills the grid (every workgroup gets a share of at least the partition)
  // keeps enough loads in flight with 4 load instructions per chunk, and the shorter chunk
  // trims the tail; a small call has few workgroups and needs the deeper chunk. Measured
  // with 2 q heads per kv head: batch 64 98.2 -> 96.4 us per call, batch 16 -2.5%, batch
  // 512 unchanged, batch 1 and 4 6-7% slower with the shorter chunk.
  const int64_t cap = (int64_t)a.max_blocks_per_seq * a.block_size;
  const bool full = (int64_t)a.num_seqs * cap >= (int64_t)a.max_workgroups * a.partition;
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return run_decode_hpw<T, D, 1, 8>(a, s);
    case 2: return full ? run_decode_hpw<T, D, 2, 4>(a, s) : run_decode_hpw<T, D, 2, 8>(a, s);
    case 4: return run_decode_hpw<T, D, 4, 4>(a, s);
    case 8: return run_decode_hpw<T, D, 8, 2>(a, s);
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
