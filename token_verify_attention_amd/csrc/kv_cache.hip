// INT8 KV quantisation and KV append kernels for gfx950.
//
// Quantisation rule ("CXL-SpecKV", Algorithm 2, steps 3 and 5; key
// observation (4)): per (token, head) row of d values,
//   a = max|x|, scale = fp16_rne(a / 127), code = clamp(rne(fp32(x / scale)), +-127),
// all codes 0 when the fp16 scale is 0.  The fp32 divisions are IEEE correctly
// rounded (HIP's default division; no fast-math anywhere in this library).
//
// Layout: a row is handled by a group of 16 lanes, each holding d/16
// consecutive values, so a wave covers 4 rows and every global access is a
// contiguous 8..64-byte chunk per lane.
#include "common.h"
#include "launch.h"
#include "kv_rows.h"

namespace sva {

constexpr int kQuantThreads = 256;
constexpr int kRowsPerBlock = kQuantThreads / kRowLanes;   // 16

template <typename Src, int D>
__global__ __launch_bounds__(kQuantThreads) void kv_quant_int8_kernel(
    const Src* __restrict__ x, int64_t rows, int8_t* __restrict__ codes,
    uint16_t* __restrict__ scales) {
  constexpr int N = D / kRowLanes;
  const int sub = threadIdx.x % kRowLanes;
  for (int64_t row = int64_t(blockIdx.x) * kRowsPerBlock + threadIdx.x / kRowLanes; row < rows;
       row += int64_t(gridDim.x) * kRowsPerBlock) {
    float v[N];
    Chunk<Src, N>::load(x + row * D + sub * N, v);
    int8_t c[N];
    const uint16_t s16 = quant_row<N>(v, c);
    store_codes<N>(codes + row * D + sub * N, c);
    if (sub == 0) scales[row] = s16;
  }
}

// ---- append ----------------------------------------------------------------

struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* k;
  void* v;
  uint16_t* k_scale;
  uint16_t* v_scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* cu_q;
  int32_t B, T, Hkv, num_pages, max_pages;
};

constexpr int kMaxLdsSeqs = 4096;

template <typename Src, typename Dst, int D>
__global__ __launch_bounds__(kQuantThreads) void kv_append_kernel(AppendParams p) {
  constexpr int N = D / kRowLanes;
  __shared__ int32_t s_cu[kMaxLdsSeqs + 1];
  __shared__ int32_t s_ctx[kMaxLdsSeqs];
  const int sub = threadIdx.x % kRowLanes;
  const int64_t n_rows = int64_t(p.T) * p.Hkv * 2;
  const int64_t stride = int64_t(gridDim.x) * kRowsPerBlock;
  const int64_t r_first = int64_t(blockIdx.x) * kRowsPerBlock + threadIdx.x / kRowLanes;
  auto src_of = [&](int64_t r) {
    return static_cast<const Src*>((r & 1) ? p.v_new : p.k_new) + (r >> 1) * D + sub * N;
  };
  // The first row's source values depend on nothing else: their load is in
  // flight while cu_q and ctx_lens are staged, so the row costs two memory
  // round trips (lengths, then the block-table entry) before its store.
  float v[N];
  if (r_first < n_rows) Chunk<Src, N>::load(src_of(r_first), v);
  for (int i = threadIdx.x; i <= p.B; i += blockDim.x) {
    s_cu[i] = p.cu_q[i];
    if (i < p.B) s_ctx[i] = p.ctx_lens[i];
  }
  __syncthreads();
  for (int64_t r = r_first; r < n_rows; r += stride) {
    if (r != r_first) Chunk<Src, N>::load(src_of(r), v);
    const int which = int(r & 1);                 // 0: K, 1: V
    const int64_t tg = r >> 1;
    const int t = int(tg / p.Hkv);
    const int g = int(tg % p.Hkv);
    // sequence of draft row t: largest b with cu_q[b] <= t
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int pos = s_ctx[b] + (t - s_cu[b]);
    const int lp = pos / kPage;
    if (pos < 0 || lp >= p.max_pages) continue;   // out of contract: skip
    const int page = p.block_table[int64_t(b) * p.max_pages + lp];
    if (page < 0 || page >= p.num_pages) continue;
    const int64_t dst_row = (int64_t(page) * p.Hkv + g) * kPage + (pos % kPage);
    if constexpr (sizeof(Dst) == 1) {
      int8_t c[N];
      const uint16_t s16 = quant_row<N>(v, c);
      int8_t* dst = static_cast<int8_t*>(which ? p.v : p.k);
      store_codes<N>(dst + dst_row * D + sub * N, c);
      if (sub == 0) (which ? p.v_scale : p.k_scale)[dst_row] = s16;
    } else {
      Dst* dst = static_cast<Dst*>(which ? p.v : p.k);
      Chunk<Dst, N>::store(dst + dst_row * D + sub * N, v);
    }
  }
}

// ---- host launchers ----------------------------------------------------------

static int grid_for_rows(int64_t rows) {
  int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 65536) blocks = 65536;
  return int(blocks < 1 ? 1 : blocks);
}

template <typename Src, int D>
static hipError_t quant_launch(const void* x, int64_t rows, int8_t* codes, uint16_t* scales,
                               hipStream_t st) {
  hipLaunchKernelGGL((kv_quant_int8_kernel<Src, D>), dim3(grid_for_rows(rows)),
                     dim3(kQuantThreads), 0, st, static_cast<const Src*>(x), rows, codes, scales);
  return hipGetLastError();
}

hipError_t launch_kv_quant_int8(const void* x, int src_dtype, int64_t rows, int d, int8_t* codes,
                                uint16_t* scales, hipStream_t st) {
  if (src_dtype == SVA_F32) {
    if (d == 64) return quant_launch<float, 64>(x, rows, codes, scales, st);
    if (d == 128) return quant_launch<float, 128>(x, rows, codes, scales, st);
    return quant_launch<float, 256>(x, rows, codes, scales, st);
  }
  if (d == 64) return quant_launch<uint16_t, 64>(x, rows, codes, scales, st);
  if (d == 128) return quant_launch<uint16_t, 128>(x, rows, codes, scales, st);
  return quant_launch<uint16_t, 256>(x, rows, codes, scales, st);
}

template <typename Src, typename Dst, int D>
static hipError_t append_launch(const AppendParams& p, hipStream_t st) {
  const int64_t rows = int64_t(p.T) * p.Hkv * 2;
  hipLaunchKernelGGL((kv_append_kernel<Src, Dst, D>), dim3(grid_for_rows(rows)),
                     dim3(kQuantThreads), 0, st, p);
  return hipGetLastError();
}

template <typename Src, typename Dst>
static hipError_t append_d(const AppendParams& p, int d, hipStream_t st) {
  if (d == 64) return append_launch<Src, Dst, 64>(p, st);
  if (d == 128) return append_launch<Src, Dst, 128>(p, st);
  return append_launch<Src, Dst, 256>(p, st);
}

template <typename Src>
static hipError_t append_dst(const AppendParams& p, int kv_dtype, int d, hipStream_t st) {
  if (kv_dtype == SVA_F32) return append_d<Src, float>(p, d, st);
  if (kv_dtype == SVA_BF16) return append_d<Src, uint16_t>(p, d, st);
  return append_d<Src, int8_t>(p, d, st);
}

hipError_t launch_kv_append(const sva_batch* batch, const void* k_new, const void* v_new,
                            int src_dtype, const sva_paged_kv* kv, hipStream_t st) {
  AppendParams p;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k = kv->k;
  p.v = kv->v;
  p.k_scale = static_cast<uint16_t*>(kv->k_scale);
  p.v_scale = static_cast<uint16_t*>(kv->v_scale);
  p.block_table = kv->block_table;
  p.ctx_lens = batch->ctx_lens;
  p.cu_q = batch->cu_q;
  p.B = batch->B;
  p.T = batch->total_q;
  p.Hkv = kv->Hkv;
  p.num_pages = kv->num_pages;
  p.max_pages = kv->max_pages_per_seq;
  if (src_dtype == SVA_F32) return append_dst<float>(p, kv->kv_dtype, kv->d, st);
  return append_dst<uint16_t>(p, kv->kv_dtype, kv->d, st);
}

}  // namespace sva
