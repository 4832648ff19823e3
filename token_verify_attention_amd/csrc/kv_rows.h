// Rows of d values held by 16-lane groups: loading and storing them in each
// cache element type, and the INT8 quantisation rule ("CXL-SpecKV",
// Algorithm 2, steps 3 and 5; key observation (4)): per (token, head) row,
//   a = max|x|, scale = fp16_rne(a / 127), code = clamp(rne(fp32(x / scale)), +-127),
// all codes 0 when the fp16 scale is 0.  Shared by the cache kernels and by
// the verification kernel's append of the new rows, so both write the same
// bytes.
#pragma once
#include "common.h"

namespace sva {

constexpr int kRowLanes = 16;

template <typename T, int N>
struct Chunk;
template <int N>
struct Chunk<float, N> {
  __device__ static void load(const float* p, float* v) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      u32x4 w = q[i];
      v[4 * i + 0] = __uint_as_float(w[0]);
      v[4 * i + 1] = __uint_as_float(w[1]);
      v[4 * i + 2] = __uint_as_float(w[2]);
      v[4 * i + 3] = __uint_as_float(w[3]);
    }
  }
  __device__ static void store(float* p, const float* v) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      u32x4 w = {__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                 __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3])};
      q[i] = w;
    }
  }
};
template <int N>
struct Chunk<uint16_t, N> {   // bf16 bit patterns
  __device__ static void load(const uint16_t* p, float* v) {
    if constexpr (N % 8 == 0) {
      const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        u32x4 w = q[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bf16_lo(w[j]);
          v[8 * i + 2 * j + 1] = bf16_hi(w[j]);
        }
      }
    } else {
      const u32x2* q = reinterpret_cast<const u32x2*>(p);
      u32x2 w = q[0];
      v[0] = bf16_lo(w[0]); v[1] = bf16_hi(w[0]);
      v[2] = bf16_lo(w[1]); v[3] = bf16_hi(w[1]);
    }
  }
  __device__ static void store(uint16_t* p, const float* v) {
    if constexpr (N % 8 == 0) {
      u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(v[8 * i + 2 * j], v[8 * i + 2 * j + 1]);
        q[i] = w;
      }
    } else {
      u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2*>(p) = w;
    }
  }
};

// Quantise one row held by a 16-lane group (N = d/16 values per lane).
// Returns the fp16 scale bits; writes the lane's N codes into `codes`.
template <int N>
__device__ __forceinline__ uint16_t quant_row(const float* v, int8_t* codes) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) a = fmaxf(a, fabsf(v[i]));
  a = row16_max(a);                 // a row is one 16-lane DPP row
  const uint16_t s16 = f32_to_f16_bits(a / 127.0f);
  const float s = f16_bits_to_f32(s16);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float c = 0.f;
    if (s != 0.f) c = fminf(fmaxf(rintf(v[i] / s), -127.f), 127.f);
    codes[i] = int8_t(int(c));
  }
  return s16;
}

template <int N>
__device__ __forceinline__ void store_codes(int8_t* dst, const int8_t* c) {
  uint32_t w[N / 4];
#pragma unroll
  for (int i = 0; i < N / 4; ++i)
    w[i] = uint32_t(uint8_t(c[4 * i])) | (uint32_t(uint8_t(c[4 * i + 1])) << 8) |
           (uint32_t(uint8_t(c[4 * i + 2])) << 16) | (uint32_t(uint8_t(c[4 * i + 3])) << 24);
  if constexpr (N == 4) {
    *reinterpret_cast<uint32_t*>(dst) = w[0];
  } else if constexpr (N == 8) {
    u32x2 x = {w[0], w[1]};
    *reinterpret_cast<u32x2*>(dst) = x;
  } else {
    u32x4 x = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(dst) = x;
  }
}

}  // namespace sva
