// Device-side KV-cache pointer management ("HeteroReason", KV Cache Management
// Unit, Fig. 7) for gfx950.
//
// Every sequence carries a triplet (valid, curr, ahead): the last verified
// context boundary, the step under verification, and the step-ahead
// speculation frontier.  One thread per sequence applies that sequence's mode:
//   Initialization  valid, curr, ahead <- arg
//   Speculation     ahead <- ahead + max(arg, 0)
//   Accept          valid <- curr, curr <- ahead
//   Rollback        curr, ahead <- valid
//   Prefix commit   valid <- min(valid + max(arg, 0), ahead); curr, ahead <- valid
// (the last is the token-level form: the first n_b drafts are accepted, the
// rest discarded).  Rejected history is dropped by moving pointers only; the
// cache rows past `valid` are overwritten by later appends.  Keeping the state
// on the device lets a verification loop commit from accept_len without a
// host round trip.
#include "common.h"
#include "launch.h"

namespace sva {

__global__ __launch_bounds__(256) void kvmu_kernel(int B, const int32_t* __restrict__ mode,
                                                   int uniform_mode,
                                                   const int32_t* __restrict__ arg,
                                                   int32_t* __restrict__ state,
                                                   int32_t* __restrict__ ctx_lens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int valid = state[3 * b], curr = state[3 * b + 1], ahead = state[3 * b + 2];
  const int m = mode ? mode[b] : uniform_mode;
  const int a = arg ? arg[b] : 0;
  switch (m) {
    case SVA_KVMU_INIT:
      valid = curr = ahead = a;
      break;
    case SVA_KVMU_SPECULATE:
      ahead += max(a, 0);
      break;
    case SVA_KVMU_ACCEPT:
      valid = curr;
      curr = ahead;
      break;
    case SVA_KVMU_ROLLBACK:
      curr = ahead = valid;
      break;
    case SVA_KVMU_PREFIX:
      valid = min(valid + max(a, 0), ahead);
      curr = ahead = valid;
      break;
    default:                                // unknown modes leave the state alone
      break;
  }
  state[3 * b] = valid;
  state[3 * b + 1] = curr;
  state[3 * b + 2] = ahead;
  if (ctx_lens) ctx_lens[b] = valid;
}

// ---- pages of the speculative history -------------------------------------
// Rejected history is dropped by the pointer moves above; its pages go back
// to a caller-owned free list once a sequence's valid pointer is final for
// the step: every logical page j with 16 j >= valid holds nothing valid, so
// its page is appended to the list and its block-table entry becomes -1.
// Before the next step appends rows at S_b .. S_b + k_b - 1, every unassigned
// logical page below S_b + k_b takes the page on top of the list.  Orders are
// fixed (sequence by sequence, logical page by logical page; pages appended
// after the list's entries and taken from its top), so the result is one
// definite array: one workgroup scans the block table in that order, each
// thread a contiguous range of entries, with a workgroup prefix sum placing
// every thread's pages.

constexpr int kPageThreads = 1024;

// Exclusive prefix sum of v over the workgroup; the total lands in *total.
__device__ __forceinline__ int workgroup_exclusive_sum(int v, int* total) {
  __shared__ int s_wave[kPageThreads / kWave];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kPageThreads / kWave; ++w) {
      const int t = s_wave[w];
      s_wave[w] = run;
      run += t;
    }
    *total = run;
  }
  __syncthreads();
  return s_wave[wave] + incl - v;
}

// This thread's contiguous range of the B x max_pages block-table entries.
__device__ __forceinline__ void entry_range(int64_t n, int64_t& e0, int64_t& e1) {
  const int64_t per = (n + kPageThreads - 1) / kPageThreads;
  e0 = min(n, int64_t(threadIdx.x) * per);
  e1 = min(n, e0 + per);
}

__global__ __launch_bounds__(kPageThreads) void kv_reclaim_pages_kernel(
    int B, const int32_t* __restrict__ valid_lens, int32_t* __restrict__ block_table,
    int max_pages, int32_t* __restrict__ free_list, int32_t* __restrict__ free_count,
    int capacity) {
  __shared__ int s_total, s_base;
  if (threadIdx.x == 0) s_base = max(*free_count, 0);
  int64_t e0, e1;
  entry_range(int64_t(B) * max_pages, e0, e1);
  auto freed = [&](int64_t e) {
    const int b = int(e / max_pages), j = int(e - int64_t(b) * max_pages);
    return int64_t(kPage) * j >= max(valid_lens[b], 0) && block_table[e] >= 0;
  };
  int n = 0;
  for (int64_t e = e0; e < e1; ++e) n += freed(e);
  const int off = workgroup_exclusive_sum(n, &s_total);   // its barriers order s_base
  int64_t idx = int64_t(s_base) + off;
  for (int64_t e = e0; e < e1; ++e) {
    if (!freed(e)) continue;
    if (idx < capacity) free_list[idx] = block_table[e];
    block_table[e] = -1;
    ++idx;
  }
  if (threadIdx.x == 0) *free_count = s_base + s_total;
}

__global__ __launch_bounds__(kPageThreads) void kv_alloc_pages_kernel(
    int B, const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ cu_q,
    int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ free_list,
    int32_t* __restrict__ free_count, int capacity) {
  __shared__ int s_total, s_avail;
  if (threadIdx.x == 0) s_avail = min(max(*free_count, 0), capacity);
  int64_t e0, e1;
  entry_range(int64_t(B) * max_pages, e0, e1);
  auto needed = [&](int64_t e) {
    const int b = int(e / max_pages), j = int(e - int64_t(b) * max_pages);
    const int64_t end = int64_t(max(ctx_lens[b], 0)) + max(cu_q[b + 1] - cu_q[b], 0);
    return int64_t(kPage) * j < end && block_table[e] < 0;
  };
  int n = 0;
  for (int64_t e = e0; e < e1; ++e) n += needed(e);
  const int off = workgroup_exclusive_sum(n, &s_total);
  const int avail = s_avail;
  int i = off;                       // this entry's place among all the needed ones
  for (int64_t e = e0; e < e1 && i < avail; ++e) {
    if (!needed(e)) continue;
    block_table[e] = free_list[avail - 1 - i];
    ++i;
  }
  if (threadIdx.x == 0) *free_count = max(avail - s_total, 0);
}

hipError_t launch_kv_reclaim_pages(int B, const int32_t* valid_lens, int32_t* block_table,
                                   int max_pages, int32_t* free_list, int32_t* free_count,
                                   int capacity, hipStream_t st) {
  hipLaunchKernelGGL(kv_reclaim_pages_kernel, dim3(1), dim3(kPageThreads), 0, st, B, valid_lens,
                     block_table, max_pages, free_list, free_count, capacity);
  return hipGetLastError();
}

hipError_t launch_kv_alloc_pages(const sva_batch* batch, int32_t* block_table, int max_pages,
                                 const int32_t* free_list, int32_t* free_count, int capacity,
                                 hipStream_t st) {
  hipLaunchKernelGGL(kv_alloc_pages_kernel, dim3(1), dim3(kPageThreads), 0, st, batch->B,
                     batch->ctx_lens, batch->cu_q, block_table, max_pages, free_list, free_count,
                     capacity);
  return hipGetLastError();
}

hipError_t launch_kvmu(int B, const int32_t* mode, int uniform_mode, const int32_t* arg,
                       int32_t* state, int32_t* ctx_lens, hipStream_t st) {
  hipLaunchKernelGGL(kvmu_kernel, dim3((B + 255) / 256), dim3(256), 0, st, B, mode, uniform_mode,
                     arg, state, ctx_lens);
  return hipGetLastError();
}

}  // namespace sva
