// Helpers shared by the acceptance kernels (greedy prefix and tree walk).
#pragma once
#include "common.h"

namespace sva {

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor(uint32_t(v), o, kWave);
  const uint32_t hi = __shfl_xor(uint32_t(v >> 32), o, kWave);
  return (uint64_t(hi) << 32) | lo;
}

// Argmax tokens of rows row0 .. row0 + n - 1 (n <= 64) from their chunk keys
// (keys[row * chunks + c]: the largest 64-bit key of chunk c, the complemented
// index in the low half): lane j reduces row j and returns its token (0 on
// lanes >= n).  A lane's loads are issued 32 at a time, so a row of up to 32
// chunks (the acceptance plan's usual maximum) costs one memory round trip.
__device__ __forceinline__ int row_tokens_from_keys(const uint64_t* __restrict__ keys, int chunks,
                                                    int64_t row0, int n) {
  constexpr int kBatch = 32;
  const int lane = lane_id();
  if (lane >= n) return 0;
  const uint64_t* kp = keys + (row0 + lane) * chunks;
  uint64_t best = 0;                        // below every real key
  for (int c0 = 0; c0 < chunks; c0 += kBatch) {
    uint64_t v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) v[i] = c0 + i < chunks ? kp[c0 + i] : 0;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) best = v[i] > best ? v[i] : best;
  }
  return int(0xffffffffu - uint32_t(best));
}

}  // namespace sva
