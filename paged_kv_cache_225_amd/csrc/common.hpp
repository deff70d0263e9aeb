// Device helpers shared by the gfx950 kernels of the paged-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ---- bf16 <-> fp32 -------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){lo, hi}, bf16x2_v));
}

// ---- element traits: a 16-byte lane chunk holds EPL elements ------------------------
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;
  __device__ __forceinline__ static void unpack(const u32x4_t& c, float* f) {
    f[0] = __uint_as_float(c.x); f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z); f[3] = __uint_as_float(c.w);
  }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
  __device__ __forceinline__ static u32x4_t nan_chunk() {
    return u32x4_t{0x7fc00000u, 0x7fc00000u, 0x7fc00000u, 0x7fc00000u};
  }
};
template <> struct Elem<__bf16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
  __device__ __forceinline__ static void unpack(const u32x4_t& c, float* f) {
    f[0] = bf16_lo(c.x); f[1] = bf16_hi(c.x); f[2] = bf16_lo(c.y); f[3] = bf16_hi(c.y);
    f[4] = bf16_lo(c.z); f[5] = bf16_hi(c.z); f[6] = bf16_lo(c.w); f[7] = bf16_hi(c.w);
  }
  __device__ __forceinline__ static void store(__bf16* p, float v) { *p = (__bf16)v; }
  __device__ __forceinline__ static u32x4_t nan_chunk() {
    return u32x4_t{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
  }
};

// ---- cross-lane reductions --------------------------------------------------------------
// DPP controls (gfx9 encoding): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror. After the four steps every lane of a 16-lane row holds the row's reduction.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 1 || LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16 ||
                LANES == 32 || LANES == 64, "power-of-two lane group");
  if constexpr (LANES >= 2) x += dpp_f<0xB1>(x);
  if constexpr (LANES >= 4) x += dpp_f<0x4E>(x);
  if constexpr (LANES >= 8) x += dpp_f<0x141>(x);
  if constexpr (LANES >= 16) x += dpp_f<0x140>(x);
  if constexpr (LANES >= 32) x += __shfl_xor(x, 16);
  if constexpr (LANES >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int LANES>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (LANES >= 2) x = fmaxf(x, dpp_f<0xB1>(x));
  if constexpr (LANES >= 4) x = fmaxf(x, dpp_f<0x4E>(x));
  if constexpr (LANES >= 8) x = fmaxf(x, dpp_f<0x141>(x));
  if constexpr (LANES >= 16) x = fmaxf(x, dpp_f<0x140>(x));
  if constexpr (LANES >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (LANES >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void store16(void* p, const u32x4_t& v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

}  // namespace pkv
