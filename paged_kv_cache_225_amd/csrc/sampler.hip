// Temperature sampling of the next token from a batch of logit rows, for gfx950.
//
// The sampler of "Nano-vLLM 代码解析" (section 4.3 采样器) and of "vLLM 学习笔记 02" divides a
// row's logits by the row's temperature, takes the softmax, divides each probability by an
// independent Exp(1) draw (clamped below at 1e-10) and returns the index of the largest
// quotient: an exponential race, which picks token i with probability softmax(l / T)_i.
// The softmax denominator is the same for every index of a row, so the winner is the index
// of the largest  s_i = l_i / T - log(max(E_i, 1e-10)) ; no exp and no row sum are needed,
// and the row is read once.
//
// Random numbers: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011). Element i of row r takes 32 bits of the output block for
// counter (i / 8, r, offset, 0) and key (seed, 0): word (i % 8) / 2, its low half for even
// i and its high half for odd i. The top 23 of those bits give u = (bits + 0.5) / 2^23 in
// (0, 1), and E = -log(u).
//
// Pass 1 (sample_chunk_kernel): a workgroup takes a contiguous chunk of one row (a
// multiple of 2048 elements); each thread handles groups of 8 consecutive elements (one
// Philox block, 16- or 32-byte loads) and keeps its best (score, index); the workgroup
// reduces them and writes its chunk's winner. Pass 2 (sample_pick_kernel): one wavefront
// per row reduces the chunk winners. Ties go to the smaller index (the first maximum).
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "paged_kv.h"

namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 8;                      // elements per Philox block
constexpr int kChunkQuantum = kThreads * kGroup;  // 2048
constexpr int kTargetWorkgroups = 1024;

struct U64x4 {
  uint64_t x[4];
};

// The 128-bit product m * x as (hi, lo), from four 32 x 32 -> 64-bit multiply-adds that
// the high and low halves share (every partial sum below fits in 64 bits). 32-bit integer
// products run at a quarter of the vector rate, so they set the kernel's time.
__device__ __forceinline__ void mulhilo64(uint64_t m, uint64_t x, uint64_t& hi, uint64_t& lo) {
  const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
  const uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32);
  const uint64_t p00 = (uint64_t)ml * xl;
  const uint64_t t = (uint64_t)ml * xh + (p00 >> 32);
  const uint64_t u = (uint64_t)mh * xl + (uint32_t)t;
  hi = (uint64_t)mh * xh + (t >> 32) + (u >> 32);
  lo = (u << 32) | (uint32_t)p00;
}

__device__ __forceinline__ U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                              uint64_t c3, uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ULL, kM1 = 0xCA5A826395121157ULL;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ULL, kW1 = 0xBB67AE8584CAA73BULL;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(kM0, c0, hi0, lo0);
    mulhilo64(kM1, c2, hi1, lo1);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += kW0;
    k1 += kW1;
  }
  return U64x4{{c0, c1, c2, c3}};
}

// winner of two (score, index) candidates: larger score, then smaller index
__device__ __forceinline__ bool better(float s, int i, float bs, int bi) {
  return s > bs || (s == bs && i < bi);
}

// Natural log of a positive, normal, finite float: the hardware base-2 log times ln 2, with
// ln 2 split in two floats and the product's rounding error kept by an fma, so the result
// stays within about an ulp also where it is small (x near 1). Denormal, zero and infinite
// inputs are not handled: the callers' arguments are never such.
__device__ __forceinline__ float log_normal(float x) {
  constexpr float kLn2Hi = 0x1.62e43p-1f;     // ln 2 rounded to float
  constexpr float kLn2Lo = -0x1.05c61p-29f;   // ln 2 - kLn2Hi, rounded to float
  const float r = __builtin_amdgcn_logf(x);   // log2(x)
  const float hi = r * kLn2Hi;
  return hi + fmaf(r, kLn2Lo, fmaf(r, kLn2Hi, -hi));
}

// u = (top 23 bits + 0.5) / 2^23 is exact in fp32 and lies in [2^-24, 1 - 2^-24], so
// E = -log(u) lies in [6e-8, 16.7]: both logs take normal arguments. E keeps ~1 ulp also
// near u = 1, where it is small and the element most likely to win (a log accurate only in
// absolute terms would lose E's relative accuracy there).
__device__ __forceinline__ float score_of(float logit, float inv_t, uint32_t bits) {
  const float u = ((float)(bits >> 9) + 0.5f) * (1.0f / 8388608.0f);
  const float e = fmaxf(-log_normal(u), 1e-10f);
  return logit * inv_t - log_normal(e);
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* f);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* f) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<__bf16>(const __bf16* p, float* f) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
template <typename T>
__device__ __forceinline__ float load1(const T* p) {
  return (float)*p;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sample_chunk_kernel(
    const T* __restrict__ logits, int64_t row_stride, int32_t vocab, int32_t chunk,
    const float* __restrict__ temperatures, uint64_t seed, uint64_t offset,
    float* __restrict__ ws_score, int32_t* __restrict__ ws_index, int32_t vec) {
  const int row = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  const int64_t c1 = min((int64_t)vocab, c0 + chunk);
  const T* lrow = logits + (int64_t)row * row_stride;
  const float inv_t = 1.0f / temperatures[row];
  float best = -INFINITY;
  int best_i = INT32_MAX;
  for (int64_t g = c0 + (int64_t)threadIdx.x * kGroup; g < c1; g += (int64_t)kThreads * kGroup) {
    const U64x4 r = philox4x64_10((uint64_t)(g / kGroup), (uint64_t)row, offset, 0, seed, 0);
    float f[kGroup];
    if (vec && g + kGroup <= c1) {
      load8<T>(lrow + g, f);
    } else {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) f[j] = g + j < c1 ? load1<T>(lrow + g + j) : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const uint64_t word = r.x[j >> 1];
      const uint32_t bits = (j & 1) ? (uint32_t)(word >> 32) : (uint32_t)word;
      const float s = score_of(f[j], inv_t, bits);
      const int idx = (int)(g + j);
      if (g + j < c1 && better(s, idx, best, best_i)) {
        best = s;
        best_i = idx;
      }
    }
  }
  // wavefront, then workgroup
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float os = __shfl_xor(best, off);
    const int oi = __shfl_xor(best_i, off);
    if (better(os, oi, best, best_i)) {
      best = os;
      best_i = oi;
    }
  }
  __shared__ float s_score[kThreads / 64];
  __shared__ int s_index[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_score[wave] = best;
    s_index[wave] = best_i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(s_score[w], s_index[w], best, best_i)) {
        best = s_score[w];
        best_i = s_index[w];
      }
    const int64_t slot = (int64_t)row * gridDim.x + blockIdx.x;
    ws_score[slot] = best;
    ws_index[slot] = best_i;
  }
}

__global__ __launch_bounds__(kThreads) void sample_pick_kernel(
    int32_t* __restrict__ tokens, int32_t num_rows, int32_t chunks,
    const float* __restrict__ ws_score, const int32_t* __restrict__ ws_index) {
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= num_rows) return;
  const int lane = threadIdx.x & 63;
  float best = -INFINITY;
  int best_i = INT32_MAX;
  for (int c = lane; c < chunks; c += 64) {
    const float s = ws_score[(int64_t)row * chunks + c];
    const int i = ws_index[(int64_t)row * chunks + c];
    if (better(s, i, best, best_i)) {
      best = s;
      best_i = i;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float os = __shfl_xor(best, off);
    const int oi = __shfl_xor(best_i, off);
    if (better(os, oi, best, best_i)) {
      best = os;
      best_i = oi;
    }
  }
  if (lane == 0) tokens[row] = best_i == INT32_MAX ? 0 : best_i;
}

// chunk length (a multiple of 2048) and chunk count per row for a call
void split(int32_t num_rows, int32_t vocab, int32_t* chunk, int32_t* chunks) {
  const int64_t quanta = ((int64_t)vocab + kChunkQuantum - 1) / kChunkQuantum;
  int64_t want = (kTargetWorkgroups + num_rows - 1) / num_rows;  // chunks per row
  if (want > quanta) want = quanta;
  if (want < 1) want = 1;
  const int64_t per = (quanta + want - 1) / want;
  *chunk = (int32_t)(per * kChunkQuantum);
  *chunks = (int32_t)((vocab + *chunk - 1) / *chunk);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" {

size_t pkv_sample_workspace_bytes(int32_t num_rows, int32_t vocab_size) {
  if (num_rows <= 0 || vocab_size <= 0) return 0;
  int32_t chunk, chunks;
  split(num_rows, vocab_size, &chunk, &chunks);
  return (size_t)num_rows * chunks * (sizeof(float) + sizeof(int32_t));
}

int pkv_sample(int32_t* tokens, const void* logits, int64_t row_stride, int32_t num_rows,
               int32_t vocab_size, pkv_dtype_t dtype, const float* temperatures, uint64_t seed,
               uint64_t offset, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_rows < 0 || vocab_size <= 0 || row_stride < vocab_size) return PKV_ERR_INVALID;
  if (num_rows > 65535) return PKV_ERR_UNSUPPORTED;  // one grid row per logit row
  if (num_rows == 0) return PKV_OK;
  if (!tokens || !logits || !temperatures) return PKV_ERR_INVALID;
  const int elem = dtype == PKV_BF16 ? 2 : 4;
  // groups of 8 elements are read as 16- or 32-byte vectors when every row starts on 16
  // bytes, element by element otherwise
  const int32_t vec = aligned16(logits) && (row_stride * elem) % 16 == 0;
  const size_t need = pkv_sample_workspace_bytes(num_rows, vocab_size);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PKV_ERR_WORKSPACE;
  int32_t chunk, chunks;
  split(num_rows, vocab_size, &chunk, &chunks);
  float* ws_score = static_cast<float*>(workspace);
  int32_t* ws_index = reinterpret_cast<int32_t*>(ws_score + (size_t)num_rows * chunks);
  const dim3 grid((unsigned)chunks, (unsigned)num_rows);
  if (dtype == PKV_BF16)
    hipLaunchKernelGGL(sample_chunk_kernel<__bf16>, grid, dim3(kThreads), 0, stream,
                       static_cast<const __bf16*>(logits), row_stride, vocab_size, chunk,
                       temperatures, seed, offset, ws_score, ws_index, vec);
  else
    hipLaunchKernelGGL(sample_chunk_kernel<float>, grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(logits), row_stride, vocab_size, chunk,
                       temperatures, seed, offset, ws_score, ws_index, vec);
  hipLaunchKernelGGL(sample_pick_kernel, dim3((unsigned)((num_rows + 3) / 4)), dim3(kThreads), 0,
                     stream, tokens, num_rows, chunks, ws_score, ws_index);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
