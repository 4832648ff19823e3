// Lossless stochastic acceptance (speculative rejection sampling) for gfx950.
//
// "Decoding Speculative Decoding from First Principles", section "How does
// this drafter maintain the same distribution of the target?": draft x at a
// position with target distribution p and drafter distribution q is accepted
// with probability min(1, p(x)/q(x)); at the first rejection the emitted token
// is sampled from the residual max(p - q, 0), renormalised; if every draft is
// accepted the +1 token is sampled from p after the last draft.  p and q are
// softmax(logits / temperature).  The random numbers are inputs: u_accept[j]
// decides draft j (accept iff u < p/q), u_sample[b] picks sequence b's emitted
// token by inverse CDF (the first index whose running weight sum exceeds u
// times the total).  A residual that is zero everywhere samples from p.
//
// Four launches, every one bound by HBM reads of logit rows:
//  1. row_stats_kernel: per (row, chunk) of every target and draft row, the
//     maximum m and sum of 2^(x c - m), c = log2(e) / temperature.
//  2. stochastic_decide_kernel: one wave per sequence combines the chunks of
//     its rows, decides each draft in the log2 domain (log2 u < log2 p(x) -
//     log2 q(x), so tiny probabilities never underflow to a wrong decision),
//     finds the first rejection with a ballot and records the row to sample.
//  3. sample_chunk_sums_kernel: per (sequence, chunk) of that row, the sums of
//     the residual weights and of p, for the whole chunk and for each
//     thread's contiguous range (16-byte loads, all in flight together).
//  4. sample_pick_kernel: one wave per sequence walks down the sums: the
//     chunk where the running sum crosses u * total, the thread range inside
//     it, then the element inside that range.
// Logits must not be NaN; -inf logits are tokens of probability zero.
#include "common.h"
#include "launch.h"

#include <algorithm>
#include <climits>

namespace sva {

constexpr int kSmThreads = 256;
constexpr int kMaxChunks = 64;              // chunk prefix in one wave
constexpr float kLog2eS = 1.4426950408889634f;

struct MS {
  float m, s;                               // maximum (log2 units) and sum of 2^(x - m)
};

__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  if (b.m == -INFINITY) return a;
  if (a.m == -INFINITY) return b;
  const float m = fmaxf(a.m, b.m);
  return MS{m, a.s * exp2f(a.m - m) + b.s * exp2f(b.m - m)};
}

__device__ __forceinline__ MS ms_wave(MS v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    MS w{__shfl_xor(v.m, o, kWave), __shfl_xor(v.s, o, kWave)};
    v = ms_merge(v, w);
  }
  return v;
}

SamplePlan plan_sample(const sva_batch* batch, int V) {
  SamplePlan p;
  p.stat_rows = 2 * batch->total_q + batch->B;
  int want = p.stat_rows > 0 ? (4096 + p.stat_rows - 1) / p.stat_rows : 1;
  const int max_chunks = (V + 4095) / 4096;
  want = std::max(1, std::min(want, max_chunks));
  int len = std::max((V + want - 1) / want, (V + kMaxChunks - 1) / kMaxChunks);
  len = (len + 3) & ~3;
  p.chunk_len = len;
  p.chunks = (V + len - 1) / len;
  // kernels 3 and 4 read only the B sampled rows: finer chunks (at least 1024
  // values) keep about 4096 workgroups in flight and the pick's last serial
  // walk short
  int sw = batch->B > 0 ? (4096 + batch->B - 1) / batch->B : 1;
  sw = std::max(1, std::min(std::min(sw, kMaxChunks), (V + 1023) / 1024));
  int sl = (V + sw - 1) / sw;
  sl = (sl + 3) & ~3;
  p.s_len = sl;
  p.s_chunks = (V + sl - 1) / sl;
  p.per = ((sl + kSmThreads - 1) / kSmThreads + 3) & ~3;    // elements per thread range
  p.stats_off = 0;
  p.rec_off = (size_t(p.stat_rows) * p.chunks * sizeof(MS) + 255) & ~size_t(255);
  p.sums_off = p.rec_off + ((size_t(batch->B) * 8 * sizeof(float) + 255) & ~size_t(255));
  p.parts_off =
      p.sums_off + ((size_t(batch->B) * p.s_chunks * 2 * sizeof(float) + 255) & ~size_t(255));
  p.total_bytes = p.parts_off + size_t(batch->B) * p.s_chunks * kSmThreads * 2 * sizeof(float);
  return p;
}

template <bool kVec4>
__global__ __launch_bounds__(kSmThreads) void row_stats_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int target_rows, int V,
    int chunks, int chunk_len, float c, MS* __restrict__ stats) {
  const int row = blockIdx.x / chunks;
  const int ch = blockIdx.x % chunks;
  const float* rp = row < target_rows ? target + int64_t(row) * V
                                      : draft + int64_t(row - target_rows) * V;
  const int begin = ch * chunk_len, end = min(V, begin + chunk_len);
  MS acc{-INFINITY, 0.f};
  if constexpr (kVec4) {
    constexpr int kBatch = 16;              // f32x4 loads in flight per thread (non-temporal:
                                            // kernel 3 re-reads only the sampled rows)
    for (int i0 = begin + 4 * threadIdx.x; i0 < end; i0 += 4 * kSmThreads * kBatch) {
      f32x4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = i0 + 4 * kSmThreads * u;
        v[u] = i < end ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rp + i))
                       : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float mx = fmaxf(fmaxf(v[u][0], v[u][1]), fmaxf(v[u][2], v[u][3])) * c;
        if (mx == -INFINITY) continue;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) s += exp2f(v[u][e] * c - mx);
        acc = ms_merge(acc, MS{mx, s});
      }
    }
  } else {
    for (int i = begin + threadIdx.x; i < end; i += kSmThreads) {
      const float x = rp[i] * c;
      if (x != -INFINITY) acc = ms_merge(acc, MS{x, 1.f});
    }
  }
  acc = ms_wave(acc);
  __shared__ MS s_part[kSmThreads / kWave];
  if (lane_id() == 0) s_part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    MS t = s_part[0];
#pragma unroll
    for (int w = 1; w < kSmThreads / kWave; ++w) t = ms_merge(t, s_part[w]);
    stats[int64_t(row) * chunks + ch] = t;
  }
}

// Per-sequence record for the sampling kernels (8 floats).
struct SampleRec {
  int trow, drow;                           // target row; draft row (-1: sample p)
  float mt, zt, md, zd;                     // row maxima (log2 units) and 1 / sums
  int pad0, pad1;
};

// The row's chunk statistics merged in chunk order; the loads of up to 16
// chunks are issued together, so a row costs one memory round trip per 16
// chunks instead of one per chunk (same merge order, same result).
__device__ __forceinline__ MS row_total(const MS* stats, int row, int chunks) {
  constexpr int kBatch = 16;
  MS t{-INFINITY, 0.f};
  const MS* rs = stats + int64_t(row) * chunks;
  for (int c0 = 0; c0 < chunks; c0 += kBatch) {
    MS v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (c0 + i < chunks) v[i] = rs[c0 + i];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (c0 + i < chunks) t = ms_merge(t, v[i]);
  }
  return t;
}

__global__ __launch_bounds__(kWave) void stochastic_decide_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int V, float c,
    const MS* __restrict__ stats, int chunks, const int32_t* __restrict__ cu_q, int T, int max_q,
    const int32_t* __restrict__ draft_ids, const float* __restrict__ u_accept,
    int32_t* __restrict__ accept_len, SampleRec* __restrict__ recs) {
  const int b = blockIdx.x;
  const int lane = lane_id();
  int q0 = cu_q[b], q1 = cu_q[b + 1];
  q0 = min(max(q0, 0), T);
  q1 = min(max(q1, q0), T);
  const int k = min(q1 - q0, max_q);
  const int B = gridDim.x;
  const int row0 = q0 + b;
  MS tt{-INFINITY, 0.f}, dd{-INFINITY, 0.f};
  if (lane <= k) tt = row_total(stats, row0 + lane, chunks);
  bool reject = false;
  if (lane < k) {
    dd = row_total(stats, T + B + q0 + lane, chunks);
    const int x = min(max(draft_ids[q0 + lane], 0), V - 1);
    const float t = target[int64_t(row0 + lane) * V + x] * c;
    const float d = draft[int64_t(q0 + lane) * V + x] * c;
    if (d == -INFINITY) {
      reject = false;                       // q(x) = 0: ratio +inf, accepted
    } else if (t == -INFINITY) {
      reject = true;                        // p(x) = 0: ratio 0, rejected
    } else {
      const float lr = (t - tt.m - __log2f(tt.s)) - (d - dd.m - __log2f(dd.s));
      reject = !(__log2f(u_accept[q0 + lane]) < lr);
    }
  }
  const uint64_t bal = __ballot(reject);
  const int n = bal ? __builtin_ctzll(bal) : k;
  const float mt = __shfl(tt.m, n, kWave), zt = __shfl(tt.s, n, kWave);
  const float md = __shfl(dd.m, n, kWave), zd = __shfl(dd.s, n, kWave);
  if (lane == 0) {
    accept_len[b] = n;
    SampleRec r;
    r.trow = row0 + n;
    r.drow = n < k ? q0 + n : -1;
    r.mt = mt;
    r.zt = 1.f / zt;
    r.md = md;
    r.zd = n < k ? 1.f / zd : 0.f;
    r.pad0 = r.pad1 = 0;
    recs[b] = r;
  }
}

// Target probability and residual weight of element v of a record's rows:
// pw = 2^(t c - mt) / Zt, rw = max(pw - 2^(d c - md) / Zd, 0), or pw when the
// record samples p.  Kernels 3 and 4 evaluate each element through this one
// function, so the running sums they compare agree bit for bit.
__device__ __forceinline__ void weight_of(const SampleRec& r, float tl, float dl, float c,
                                          float& pw, float& rw) {
  pw = exp2f(tl * c - r.mt) * r.zt;
  rw = r.drow < 0 ? pw : fmaxf(pw - exp2f(dl * c - r.md) * r.zd, 0.f);
}

// Elements [a0, a1) of the sampled rows, summed in order: the thread's share
// of a chunk.  16-byte loads when the rows allow them, all issued before use.
template <bool kVec4>
__device__ __forceinline__ void range_sums(const SampleRec& r, const float* target,
                                           const float* draft, int V, float c, int a0, int a1,
                                           float& sp, float& sr) {
  const float* tp = target + int64_t(r.trow) * V;
  const float* dp = r.drow >= 0 ? draft + int64_t(r.drow) * V : tp;
  sp = 0.f;
  sr = 0.f;
  if constexpr (kVec4) {
    constexpr int kBatch = 4;                 // f32x4 loads in flight per row
    for (int v0 = a0; v0 < a1; v0 += 4 * kBatch) {
      f32x4 tv[kBatch], dv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int v = v0 + 4 * u;
        if (v < a1) {
          tv[u] = *reinterpret_cast<const f32x4*>(tp + v);
          dv[u] = *reinterpret_cast<const f32x4*>(dp + v);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (v0 + 4 * u + e < a1) {
            float pw, rw;
            weight_of(r, tv[u][e], dv[u][e], c, pw, rw);
            sp += pw;
            sr += rw;
          }
        }
      }
    }
  } else {
    for (int v = a0; v < a1; ++v) {
      float pw, rw;
      weight_of(r, tp[v], dp[v], c, pw, rw);
      sp += pw;
      sr += rw;
    }
  }
}

// Each thread owns a contiguous range of `per` elements of the chunk (a
// multiple of 4); its two sums go to `parts`, the chunk's to `sums`.
template <bool kVec4>
__global__ __launch_bounds__(kSmThreads) void sample_chunk_sums_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int V, float c,
    const SampleRec* __restrict__ recs, int chunks, int chunk_len, int per,
    float* __restrict__ sums, float* __restrict__ parts) {
  const int b = blockIdx.x / chunks;
  const int ch = blockIdx.x % chunks;
  const SampleRec r = recs[b];
  const int begin = ch * chunk_len, end = min(V, begin + chunk_len);
  const int a0 = min(end, begin + threadIdx.x * per), a1 = min(end, a0 + per);
  float sp, sr;
  range_sums<kVec4>(r, target, draft, V, c, a0, a1, sp, sr);
  const int64_t pi = ((int64_t(b) * chunks + ch) * kSmThreads + threadIdx.x) * 2;
  parts[pi] = sr;
  parts[pi + 1] = sp;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    sp += __shfl_xor(sp, o, kWave);
    sr += __shfl_xor(sr, o, kWave);
  }
  __shared__ float s_p[kSmThreads / kWave], s_r[kSmThreads / kWave];
  if (lane_id() == 0) {
    s_p[threadIdx.x / kWave] = sp;
    s_r[threadIdx.x / kWave] = sr;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 0.f, e = 0.f;
    for (int w = 0; w < kSmThreads / kWave; ++w) {
      a += s_r[w];
      e += s_p[w];
    }
    sums[(int64_t(b) * chunks + ch) * 2] = a;
    sums[(int64_t(b) * chunks + ch) * 2 + 1] = e;
  }
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ float wave_prefix(float x) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const float y = __shfl_up(x, o, kWave);
    if (lane_id() >= o) x += y;
  }
  return x;
}

// The first of `n` <= 64 lane values (lane i: w_i, inclusive prefix incl_i)
// whose prefix exceeds goal; when rounding leaves none, the last non-zero one.
__device__ __forceinline__ int first_over(float w, float incl, float goal, int n) {
  const int lane = lane_id();
  const uint64_t over = __ballot(lane < n && incl > goal);
  const uint64_t nz = __ballot(lane < n && w > 0.f);
  return over ? __builtin_ctzll(over) : (nz ? 63 - __builtin_clzll(nz) : 0);
}

// One wave per sequence: the chunk, then the thread range, then the element
// where the running sum first exceeds u * total.
template <bool kVec4>
__global__ __launch_bounds__(kWave) void sample_pick_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int V, float c,
    const SampleRec* __restrict__ recs, int chunks, int chunk_len, int per,
    const float* __restrict__ sums, const float* __restrict__ parts,
    const float* __restrict__ u_sample, int32_t* __restrict__ next_token) {
  const int b = blockIdx.x;
  const int lane = lane_id();
  const SampleRec r = recs[b];
  // 1. chunks: residual weights unless all are zero (then p)
  const float rs = lane < chunks ? sums[(int64_t(b) * chunks + lane) * 2] : 0.f;
  float rt = rs;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) rt += __shfl_xor(rt, o, kWave);
  const int sel = (r.drow >= 0 && rt > 0.f) ? 0 : 1;
  const float wc = lane < chunks ? sums[(int64_t(b) * chunks + lane) * 2 + sel] : 0.f;
  const float ic = wave_prefix(wc);
  const float total = __shfl(ic, kWave - 1, kWave);
  float goal = fminf(fmaxf(u_sample[b], 0.f), 1.f) * total;
  const int ch = first_over(wc, ic, goal, chunks);
  goal -= __shfl(ic - wc, ch, kWave);
  // 2. the chunk's thread ranges, four per lane
  const float* pp = parts + (int64_t(b) * chunks + ch) * kSmThreads * 2;
  float w4[4], s4 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w4[i] = pp[(4 * lane + i) * 2 + sel];
    s4 += w4[i];
  }
  const float i4 = wave_prefix(s4);
  const int lq = first_over(s4, i4, goal, kWave);
  goal -= __shfl(i4 - s4, lq, kWave);
  // within lane lq's four ranges: the first whose running sum exceeds goal
  // (rounding may leave none: then the last one of non-zero weight)
  int ti = -1, last = -1;
  float pre = 0.f, pre_at = 0.f, pre_last = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float wi = __shfl(w4[i], lq, kWave);
    if (ti < 0 && wi > 0.f && pre + wi > goal) {
      ti = i;
      pre_at = pre;
    }
    if (wi > 0.f) {
      last = i;
      pre_last = pre;
    }
    pre += wi;
  }
  if (ti < 0) {
    ti = last >= 0 ? last : 0;
    pre_at = last >= 0 ? pre_last : 0.f;
  }
  const int t = 4 * lq + ti;
  goal -= pre_at;
  // 3. the elements of thread range t: loaded by the whole wave at once, then
  // summed in element order (as the range's partial was) through shuffles
  const int begin = ch * chunk_len, end = min(V, begin + chunk_len);
  const int a0 = min(end, begin + t * per), a1 = min(end, a0 + per);
  const float* tp = target + int64_t(r.trow) * V;
  const float* dp = r.drow >= 0 ? draft + int64_t(r.drow) * V : tp;
  float acc = 0.f;
  int pick = -1, nz = -1;
  for (int base = a0; base < a1 && pick < 0; base += kWave) {
    const int v = base + lane;
    float w = 0.f;
    if (v < a1) {
      float pw, rw;
      weight_of(r, tp[v], dp[v], c, pw, rw);
      w = sel ? pw : rw;
    }
    const int m = min(kWave, a1 - base);
    for (int i = 0; i < m; ++i) {
      const float wi = __shfl(w, i, kWave);
      acc += wi;
      if (wi > 0.f) {
        nz = base + i;
        if (acc > goal) {
          pick = base + i;
          break;
        }
      }
    }
  }
  if (lane == 0) next_token[b] = pick >= 0 ? pick : (nz >= 0 ? nz : a0);
}

hipError_t launch_accept_stochastic(const sva_batch* batch, const float* target_logits,
                                    const float* draft_logits, int V, float temperature,
                                    const int32_t* draft_ids, const float* u_accept,
                                    const float* u_sample, int32_t* accept_len,
                                    int32_t* next_token, const SamplePlan& plan, void* workspace,
                                    hipStream_t st) {
  char* ws = static_cast<char*>(workspace);
  MS* stats = reinterpret_cast<MS*>(ws + plan.stats_off);
  SampleRec* recs = reinterpret_cast<SampleRec*>(ws + plan.rec_off);
  float* sums = reinterpret_cast<float*>(ws + plan.sums_off);
  float* parts = reinterpret_cast<float*>(ws + plan.parts_off);
  const float c = kLog2eS / temperature;
  const int T = batch->total_q, B = batch->B;
  const bool vec4 = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(target_logits) & 15) == 0) &&
                    (T == 0 || (reinterpret_cast<uintptr_t>(draft_logits) & 15) == 0);
  const dim3 g1(unsigned(plan.stat_rows) * plan.chunks);
  if (vec4)
    hipLaunchKernelGGL(row_stats_kernel<true>, g1, dim3(kSmThreads), 0, st, target_logits,
                       draft_logits, T + B, V, plan.chunks, plan.chunk_len, c, stats);
  else
    hipLaunchKernelGGL(row_stats_kernel<false>, g1, dim3(kSmThreads), 0, st, target_logits,
                       draft_logits, T + B, V, plan.chunks, plan.chunk_len, c, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stochastic_decide_kernel, dim3(B), dim3(kWave), 0, st, target_logits,
                     draft_logits, V, c, stats, plan.chunks, batch->cu_q, T, batch->max_q,
                     draft_ids, u_accept, accept_len, recs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 g3(unsigned(B) * plan.s_chunks);
  if (vec4) {
    hipLaunchKernelGGL(sample_chunk_sums_kernel<true>, g3, dim3(kSmThreads), 0, st,
                       target_logits, draft_logits, V, c, recs, plan.s_chunks, plan.s_len,
                       plan.per, sums, parts);
  } else {
    hipLaunchKernelGGL(sample_chunk_sums_kernel<false>, g3, dim3(kSmThreads), 0, st,
                       target_logits, draft_logits, V, c, recs, plan.s_chunks, plan.s_len,
                       plan.per, sums, parts);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (vec4) {
    hipLaunchKernelGGL(sample_pick_kernel<true>, dim3(B), dim3(kWave), 0, st, target_logits,
                       draft_logits, V, c, recs, plan.s_chunks, plan.s_len, plan.per, sums,
                       parts, u_sample, next_token);
  } else {
    hipLaunchKernelGGL(sample_pick_kernel<false>, dim3(B), dim3(kWave), 0, st, target_logits,
                       draft_logits, V, c, recs, plan.s_chunks, plan.s_len, plan.per, sums,
                       parts, u_sample, next_token);
  }
  return hipGetLastError();
}

}  // namespace sva
