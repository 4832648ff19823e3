// Greedy longest-prefix acceptance for gfx950.
//
// "Decoding Speculative Decoding from First Principles", section "Speculating
// to get sequence parallelism during decode": the target's token at each
// verified position is compared with the draft; the first disagreement stops
// acceptance and the target's token there (or the bonus token after the last
// draft) is emitted.  Greedy reading: the target's token is the row argmax.
//
// Kernel 1 streams the logits once (HBM bound): every workgroup scans one
// chunk of one row with 16-byte loads and reduces to a single 64-bit key
//   key = (order-preserving float bits << 32) | (0xffffffff - index)
// so that the maximum key is the maximum value with the lowest index among
// ties.  NaN maps to the top key (first NaN wins) and -0.0 to +0.0.
// Kernel 2 runs one wave per sequence: lane j reduces the chunk keys of the
// sequence's row j (all of a row's keys loaded together) and keeps its token,
// and a ballot finds the first draft that disagrees.
#include "common.h"
#include "launch.h"
#include "accept_keys.h"

namespace sva {

constexpr int kArgThreads = 256;

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0xffffffffu;           // NaN: the maximum
  if (f == 0.f) f = 0.f;                    // -0.0 compares equal to +0.0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float f, uint32_t idx) {
  return (uint64_t(order_key(f)) << 32) | uint64_t(0xffffffffu - idx);
}


template <bool kVec4>
__global__ __launch_bounds__(kArgThreads) void argmax_chunks_kernel(
    const float* __restrict__ logits, int V, int chunks, int chunk_len,
    uint64_t* __restrict__ keys) {
  const int row = blockIdx.x / chunks;
  const int ch = blockIdx.x % chunks;
  const int begin = ch * chunk_len;
  const int end = min(V, begin + chunk_len);
  const float* rp = logits + int64_t(row) * V;
  uint64_t best = 0;                        // below every real key
  if constexpr (kVec4) {
    // begin, chunk_len and V are multiples of 4 and rows are 16-byte aligned;
    // sixteen 16-byte loads in flight per thread (a 16K-value chunk in one
    // round), non-temporal (the logits are read once)
    constexpr int kBatch = 16;
    for (int i0 = begin + 4 * threadIdx.x; i0 < end; i0 += 4 * kArgThreads * kBatch) {
      f32x4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = i0 + 4 * kArgThreads * u;
        if (i < end) v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rp + i));
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = i0 + 4 * kArgThreads * u;
        if (i >= end) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint64_t k = make_key(v[u][e], uint32_t(i + e));
          best = k > best ? k : best;
        }
      }
    }
  } else {
    for (int i = begin + threadIdx.x; i < end; i += kArgThreads) {
      const uint64_t k = make_key(rp[i], uint32_t(i));
      best = k > best ? k : best;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const uint64_t other = shfl_xor_u64(best, o);
    best = other > best ? other : best;
  }
  __shared__ uint64_t s_best[kArgThreads / kWave];
  if (lane_id() == 0) s_best[threadIdx.x / kWave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t b = s_best[0];
#pragma unroll
    for (int w = 1; w < kArgThreads / kWave; ++w) b = s_best[w] > b ? s_best[w] : b;
    keys[int64_t(row) * chunks + ch] = b;
  }
}

__global__ __launch_bounds__(kWave) void accept_scan_kernel(
    const uint64_t* __restrict__ keys, int chunks, const int32_t* __restrict__ cu_q, int T,
    int max_q, const int32_t* __restrict__ draft_ids, int32_t* __restrict__ argmax_ids,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ next_token) {
  const int b = blockIdx.x;
  const int lane = lane_id();
  int q0 = cu_q[b], q1 = cu_q[b + 1];
  q0 = min(max(q0, 0), T);
  q1 = min(max(q1, q0), T);
  const int k = min(q1 - q0, max_q);        // k <= 16 < 64 lanes
  const int row0 = q0 + b;
  const int draft = lane < k ? draft_ids[q0 + lane] : 0;
  const int tok = row_tokens_from_keys(keys, chunks, row0, k + 1);   // lane j: row j
  if (lane <= k) argmax_ids[row0 + lane] = tok;
  const bool mismatch = lane < k && draft != tok;
  const uint64_t bal = __ballot(mismatch);
  const int n = bal ? __builtin_ctzll(bal) : k;
  const int nxt = __shfl(tok, n, kWave);
  if (lane == 0) {
    accept_len[b] = n;
    next_token[b] = nxt;
  }
}

AcceptPlan plan_accept(const sva_batch* batch, int V) {
  AcceptPlan p;
  p.rows = batch->total_q + batch->B;
  // about 6144 workgroups, each chunk at least 4096 values (against 3072:
  // ragged-batch step 437.5 -> 435.0 us, 8B GQA 122.7 -> 121.1 us in A/B)
  int want = p.rows > 0 ? (6144 + p.rows - 1) / p.rows : 1;
  const int max_chunks = (V + 4095) / 4096;
  if (want > max_chunks) want = max_chunks;
  if (want < 1) want = 1;
  int len = (V + want - 1) / want;
  len = (len + 3) & ~3;
  p.chunk_len = len;
  p.chunks = (V + len - 1) / len;
  p.total_bytes = size_t(p.rows) * p.chunks * sizeof(uint64_t);
  return p;
}

hipError_t launch_argmax_keys(const float* logits, int V, const AcceptPlan& plan,
                              uint64_t* keys, hipStream_t st) {
  const bool vec4 = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  const dim3 grid(unsigned(plan.rows) * plan.chunks);
  if (vec4)
    hipLaunchKernelGGL(argmax_chunks_kernel<true>, grid, dim3(kArgThreads), 0, st, logits, V,
                       plan.chunks, plan.chunk_len, keys);
  else
    hipLaunchKernelGGL(argmax_chunks_kernel<false>, grid, dim3(kArgThreads), 0, st, logits, V,
                       plan.chunks, plan.chunk_len, keys);
  return hipGetLastError();
}

hipError_t launch_accept_prefix(const sva_batch* batch, const float* logits, int V,
                                const int32_t* draft_ids, int32_t* argmax_ids, int32_t* accept_len,
                                int32_t* next_token, const AcceptPlan& plan, void* workspace,
                                hipStream_t st) {
  uint64_t* keys = static_cast<uint64_t*>(workspace);
  hipError_t e = launch_argmax_keys(logits, V, plan, keys, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_scan_kernel, dim3(batch->B), dim3(kWave), 0, st, keys, plan.chunks,
                     batch->cu_q, batch->total_q, batch->max_q, draft_ids, argmax_ids, accept_len,
                     next_token);
  return hipGetLastError();
}

}  // namespace sva
