// Streaming-read probe for gfx950: the rate at which one kernel can read HBM
// on this device -- the achievable ceiling of the verification kernel's KV
// stream, which reads every KV byte once ("Decoding Speculative Decoding from
// First Principles", prerequisite section on the roofline: a decode step is
// bound by reading the cache from memory, not by its arithmetic).  It is a
// measurement utility, not a step of the method.
//
// The buffer is read once with non-temporal 16-byte loads; workgroup w takes
// the contiguous range [w n / W, (w+1) n / W) of its 1 KB blocks.
//   mode 0  into registers: every thread keeps kInflight loads in flight and
//           folds them into one word per wave (written to `sink`, so no load
//           is dead);
//   mode 1  global -> LDS copies (global_load_lds_dwordx4, the path the
//           verification kernel streams pages through): each wave issues one
//           1 KB copy per instruction and keeps up to kRingKB of them in
//           flight; nothing reads the LDS;
//   mode 2  as mode 1 over 4 KB pages taken in a scattered order -- the
//           access pattern of a paged KV cache whose pages lie anywhere in
//           memory: with n = bytes / 4096 pages (a power of two), position j
//           of the order is page (j * kPageMul) mod n, a permutation since
//           kPageMul is odd, and workgroup w takes positions
//           [w n / W, (w+1) n / W).
#include "common.h"
#include "launch.h"

namespace sva {

constexpr int kProbeThreads = 256;
constexpr int kProbeWaves = kProbeThreads / kWave;
constexpr int kInflight = 8;
constexpr int kRingKB = 32;
constexpr uint64_t kPageMul = 0x9E3779B97F4A7C15ull;    // odd

__device__ __forceinline__ uint32_t fold4(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__global__ __launch_bounds__(kProbeThreads) void stream_read_regs_kernel(
    const u32x4* __restrict__ src, int64_t nkb, uint32_t* __restrict__ sink) {
  const int W = gridDim.x;
  const int64_t b0 = nkb * blockIdx.x / W * 64, b1 = nkb * (blockIdx.x + 1) / W * 64;
  uint32_t acc = 0;
  for (int64_t i0 = b0 + threadIdx.x; i0 < b1; i0 += int64_t(kProbeThreads) * kInflight) {
    u32x4 v[kInflight];
#pragma unroll
    for (int u = 0; u < kInflight; ++u) {
      const int64_t i = i0 + int64_t(kProbeThreads) * u;
      v[u] = i < b1 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kInflight; ++u) acc ^= fold4(v[u]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  if (lane_id() == 0) sink[blockIdx.x * kProbeWaves + threadIdx.x / kWave] = acc;
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* l) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)l));
}

__global__ __launch_bounds__(kProbeThreads) void stream_read_lds_kernel(
    const char* __restrict__ src, int64_t nkb, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) char ring[kProbeWaves][kRingKB][1024];
  const int W = gridDim.x;
  const int64_t c0 = nkb * blockIdx.x / W, c1 = nkb * (blockIdx.x + 1) / W;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const uint32_t off = uint32_t(lane_id()) * 16;
  int slot = 0;
  for (int64_t c = c0 + wave; c < c1; c += kProbeWaves) {
    const char* base = src + c * 1024;           // wave-uniform
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 ::"v"(off), "s"(base), "s"(lds_addr_of(ring[wave][slot])) : "memory", "m0");
    slot = slot + 1 == kRingKB ? 0 : slot + 1;
    // at most kRingKB copies in flight (the ring's slots are never read)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRingKB - 1) : "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x < kWave)
    sink[blockIdx.x * kProbeWaves + threadIdx.x / kWave] =
        *reinterpret_cast<const uint32_t*>(&ring[0][0][4 * lane_id()]);
}

__global__ __launch_bounds__(kProbeThreads) void stream_read_pages_kernel(
    const char* __restrict__ src, int64_t npages, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) char ring[kProbeWaves][kRingKB][1024];
  const int W = gridDim.x;
  const int64_t p0 = npages * blockIdx.x / W, p1 = npages * (blockIdx.x + 1) / W;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const uint32_t off = uint32_t(lane_id()) * 16;
  const uint64_t mask = uint64_t(npages) - 1;
  int slot = 0;
  // wave v reads 1 KB quarter (c mod 4) of the pages in turn (kProbeWaves = 4)
  for (int64_t c = 4 * p0 + wave; c < 4 * p1; c += kProbeWaves) {
    const uint64_t page = (uint64_t(c >> 2) * kPageMul) & mask;   // wave-uniform
    const char* base = src + page * 4096 + (c & 3) * 1024;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 ::"v"(off), "s"(base), "s"(lds_addr_of(ring[wave][slot])) : "memory", "m0");
    slot = slot + 1 == kRingKB ? 0 : slot + 1;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRingKB - 1) : "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x < kWave)
    sink[blockIdx.x * kProbeWaves + threadIdx.x / kWave] =
        *reinterpret_cast<const uint32_t*>(&ring[0][0][4 * lane_id()]);
}
static_assert(kProbeWaves == 4, "the page kernel's waves take the four 1 KB quarters of a page");

hipError_t launch_stream_read_probe(const void* buf, size_t bytes, int mode, int num_wg,
                                    uint32_t* sink, hipStream_t st) {
  const int64_t nkb = int64_t(bytes / 1024);
  if (mode == 0)
    hipLaunchKernelGGL(stream_read_regs_kernel, dim3(num_wg), dim3(kProbeThreads), 0, st,
                       static_cast<const u32x4*>(buf), nkb, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(stream_read_lds_kernel, dim3(num_wg), dim3(kProbeThreads), 0, st,
                       static_cast<const char*>(buf), nkb, sink);
  else
    hipLaunchKernelGGL(stream_read_pages_kernel, dim3(num_wg), dim3(kProbeThreads), 0, st,
                       static_cast<const char*>(buf), nkb / 4, sink);
  return hipGetLastError();
}

}  // namespace sva
