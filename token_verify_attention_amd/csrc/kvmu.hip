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

hipError_t launch_kvmu(int B, const int32_t* mode, int uniform_mode, const int32_t* arg,
                       int32_t* state, int32_t* ctx_lens, hipStream_t st) {
  hipLaunchKernelGGL(kvmu_kernel, dim3((B + 255) / 256), dim3(256), 0, st, B, mode, uniform_mode,
                     arg, state, ctx_lens);
  return hipGetLastError();
}

}  // namespace sva
