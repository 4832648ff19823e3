// Device helpers shared by the gfx950 kernels of libspecverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sva {

constexpr int kWave = 64;
constexpr int kPage = 16;

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

// ---- bf16 / fp16 conversions (bit level, exact where stated) -------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even (gfx950's v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// Two floats as packed fp16, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
// Element-wise product of two packed fp16 pairs (v_pk_mul_f16).
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) * __builtin_bit_cast(f16x2_t, b));
}
// Half `hi` of a packed fp16 pair, widened to fp32 (folds into v_fma_mix_f32).
__device__ __forceinline__ float f16x2_half(uint32_t w, int hi) {
  return float(__builtin_bit_cast(f16x2_t, w)[hi]);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return float(__builtin_bit_cast(_Float16, h));
}
// fp32 -> fp16 round to nearest even (v_cvt_f16_f32 under the default mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// ---- wave-level reductions -------------------------------------------------
// All-reduce within each 16-lane row with DPP (quad swaps, half-row mirror,
// row mirror), then across rows with gfx950's permlane16/32 swaps; every lane
// receives the result.  No LDS traffic.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));   // row_mirror
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}
// v_permlane16_swap / v_permlane32_swap exchange rows between two registers
// (odd 16-lane rows of the first with even rows of the second; the upper half
// of the first with the lower half of the second).  The results are taken out
// of the builtin's pair by value: bit-casting an element of the pair in place
// makes this compiler read the first element twice.
// For every lane: (its value, the value of the same lane in the partner row),
// rows paired (0,1), (2,3).
__device__ __forceinline__ void xrow16_pair(float v, float& a, float& b) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
// Same across the two 32-lane halves of the wave.
__device__ __forceinline__ void xrow32_pair(float v, float& a, float& b) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float xrow16_max(float v) {
  float a, b;
  xrow16_pair(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xrow16_sum(float v) {
  float a, b;
  xrow16_pair(v, a, b);
  return a + b;
}
__device__ __forceinline__ float xrow32_max(float v) {
  float a, b;
  xrow32_pair(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xrow32_sum(float v) {
  float a, b;
  xrow32_pair(v, a, b);
  return a + b;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Read a wave-uniform value from one lane into a scalar register.
__device__ __forceinline__ int readlane(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

}  // namespace sva
