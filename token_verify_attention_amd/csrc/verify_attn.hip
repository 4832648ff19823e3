// Causal multi-query verification attention over a paged KV cache, gfx950.
//
// What is computed ("Decoding Speculative Decoding from First Principles",
// section "Speculating to get sequence parallelism during decode"; "CXL-SpecKV",
// key observation (1)): for sequence b, draft query i and query head h (kv head
// g = h / G), softmax(scale * q . K_p) V_p over positions p = 0 .. S_b + i.
// Split-KV with an online softmax reaches exactly that result; every partial
// carries (running max m, weight sum l, unnormalised output O).
//
// Work decomposition.  The pages of all (sequence, kv-head) pairs are laid end
// to end; workgroup w streams the contiguous range [w*N/W, (w+1)*N/W) of
// that list, which may cover the tail of one pair, whole pairs and the head of
// another.  Every (b, g) segment is processed by the 4 waves of the workgroup,
// each taking every 4th page, so the k_b*G query rows of the pair share each
// K/V page load (the point of verification: one KV read amortised over all
// drafts, same page, "Decoding Speculative Decoding...", sequence-parallel
// section).  Waves merge through LDS.  A pair that spans several workgroups
// leaves partials in the workspace; the last workgroup to finish the pair
// (device-scope counter) merges them, so the whole call is one kernel.
//
// Per-wave inner loops:
//  * VALU path (k_b*G < 16): K and V pages staged in LDS; lane = (token,
//    quarter of d); fp32 dot products, online softmax over 16-lane groups,
//    P.V with each lane owning d/64 output columns.
//  * MFMA path (k_b*G >= 16, bf16 or INT8 cache): S^T = K Q^T with
//    v_mfma_f32_16x16x32_bf16 (K rows loaded straight into the A operand),
//    softmax in the MFMA output layout (a lane owns one query row and 4
//    tokens), O^T += V^T P^T with v_mfma_f32_16x16x16_bf16, V^T read from a
//    swizzled LDS copy of the page.  INT8 codes convert exactly to bf16; the
//    per-token scales multiply the score (K) and the probability (V).
//
// Positions at or past S_b + k_b (garbage slots of the last page) are masked
// in the scores and zeroed in V, so NaN garbage never reaches an output.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace sva {

constexpr int kAttnThreads = 256;
constexpr int kWaves = kAttnThreads / kWave;   // 4
constexpr int kMaxB = 4096;
constexpr int kMfmaRows = 32;
constexpr int kValuRows = 16;
constexpr float kNegBig = -1.0e30f;            // finite start value of running maxima
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* cu_q;
  void* out;
  float* partials;
  int32_t* counters;
  float scale_log2;     // softmax_scale * log2(e)
  int q_f32, out_f32;
  int B, T, Hq, Hkv, G, num_pages, max_pages, max_q;
  int slot_rows;        // rows per partial slot (max_q * G)
  int W;                // grid size
  int path;             // 0 auto, 1 VALU, 2 MFMA
};

struct SeqInfo {
  int S, k, q0, np;
};

// Sequence b with every device-resident value clamped into the buffers.
__device__ __forceinline__ SeqInfo seq_info(const AttnParams& p, int b) {
  int q0 = p.cu_q[b], q1 = p.cu_q[b + 1];
  q0 = min(max(q0, 0), p.T);
  q1 = min(max(q1, q0), p.T);
  SeqInfo s;
  s.q0 = q0;
  s.k = min(q1 - q0, p.max_q);
  s.S = max(p.ctx_lens[b], 0);
  s.np = 0;
  if (s.k > 0) {
    const int64_t need = (int64_t(s.S) + s.k + kPage - 1) / kPage;
    s.np = int(min(need, int64_t(p.max_pages)));
  }
  return s;
}

struct Seg {
  int b, g, S, k, q0, np;
  int pa, pe;     // page range within the pair
  int R;          // query rows of the pair: k * G
  bool full;      // the segment is the whole pair
  int slot;       // partial slot when !full
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int clamp_page(int pid, int num_pages) {
  return min(max(pid, 0), num_pages - 1);
}

// Page ids of pages j0, j0+4, ..., one per lane (0 past `pe`).
__device__ __forceinline__ int load_page_ids(const AttnParams& p, const Seg& sg, int j0) {
  const int j = j0 + kWaves * lane_id();
  int pid = 0;
  if (j < sg.pe) pid = p.block_table[int64_t(sg.b) * p.max_pages + j];
  return clamp_page(pid, p.num_pages);
}

// Element offset of (page, kv head g) in a [P, Hkv, 16, D] pool.
template <int D>
__device__ __forceinline__ int64_t page_off(const AttnParams& p, int pid, int g) {
  return (int64_t(pid) * p.Hkv + g) * (kPage * D);
}

// Output / partial-slot addressing -------------------------------------------

__device__ __forceinline__ int64_t out_row(const AttnParams& p, const Seg& sg, int r) {
  const int i = r / p.G;
  const int j = r - i * p.G;
  return (int64_t(sg.q0 + i) * p.Hq + sg.g * p.G + j);
}

template <int D>
__device__ __forceinline__ float* slot_base(const AttnParams& p, int slot) {
  return p.partials + int64_t(slot) * p.slot_rows * (D + 2);
}

__device__ __forceinline__ void store_out4(const AttnParams& p, int64_t elem, f32x4 v) {
  if (p.out_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + elem) = v;
  } else {
    u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + elem) = w;
  }
}
__device__ __forceinline__ void store_out1(const AttnParams& p, int64_t elem, float v) {
  if (p.out_f32) static_cast<float*>(p.out)[elem] = v;
  else static_cast<uint16_t*>(p.out)[elem] = f32_to_bf16(v);
}

// ============================================================================
// MFMA path
// ============================================================================

// 8 consecutive Q values as bf16 (fp32 Q rounds to nearest even).
__device__ __forceinline__ bf16x8 load_q8_bf16(const AttnParams& p, int64_t elem) {
  u32x4 w;
  if (p.q_f32) {
    const f32x4* s = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) + elem);
    const f32x4 a = s[0], b = s[1];
    w[0] = pack_bf16x2(a[0], a[1]);
    w[1] = pack_bf16x2(a[2], a[3]);
    w[2] = pack_bf16x2(b[0], b[1]);
    w[3] = pack_bf16x2(b[2], b[3]);
  } else {
    w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) + elem);
  }
  return __builtin_bit_cast(bf16x8, w);
}

// Two int8 codes (low 16 bits of w >> sh) as packed bf16 -- exact: |code| <= 127.
__device__ __forceinline__ uint32_t codes2_to_bf16x2(uint32_t w, int sh) {
  const float a = float(int(w << (24 - sh)) >> 24);
  const float b = float(int(w << (16 - sh)) >> 24);
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// 16 int8 codes (one 16-byte word) -> 16 bf16 (two 16-byte words).
__device__ __forceinline__ void codes16_to_bf16(u32x4 c, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    lo[2 * e] = codes2_to_bf16x2(c[e], 0);
    lo[2 * e + 1] = codes2_to_bf16x2(c[e], 16);
    hi[2 * e] = codes2_to_bf16x2(c[2 + e], 0);
    hi[2 * e + 1] = codes2_to_bf16x2(c[2 + e], 16);
  }
}

// Registers holding one page for one wave (MFMA path).
//  K: lane (l16, c) holds row l16, d in [c*D/4, (c+1)*D/4)  (D/4 values)
//  V: 16-byte chunks id = lane + 64*e of the page in row-major order
template <typename KV, int D>
struct MfmaPage {
  static constexpr int KBYTES = (D / 4) * int(sizeof(KV));   // per lane
  static constexpr int KCH = KBYTES / 16;                    // 16-byte loads for K
  static constexpr int VCH = kPage * D * int(sizeof(KV)) / 16 / kWave;
  u32x4 k[KCH];
  u32x4 v[VCH];
  f32x4 ksc, vsc;                                            // INT8: tokens 4c..4c+3 (unused otherwise)
};

template <typename KV, int D>
__device__ __forceinline__ void mfma_load_page(const AttnParams& p, int pid, int g,
                                               MfmaPage<KV, D>& pg) {
  const int lane = lane_id(), l16 = lane & 15, c = lane >> 4;
  const int64_t off = page_off<D>(p, pid, g);
  const KV* kb = static_cast<const KV*>(p.k) + off;
  const KV* vb = static_cast<const KV*>(p.v) + off;
  const u32x4* kp = reinterpret_cast<const u32x4*>(kb + l16 * D + c * (D / 4));
#pragma unroll
  for (int e = 0; e < MfmaPage<KV, D>::KCH; ++e) pg.k[e] = kp[e];
  const u32x4* vp = reinterpret_cast<const u32x4*>(vb);
#pragma unroll
  for (int e = 0; e < MfmaPage<KV, D>::VCH; ++e) pg.v[e] = vp[lane + kWave * e];
  if constexpr (sizeof(KV) == 1) {
    const int64_t so = (int64_t(pid) * p.Hkv + g) * kPage + 4 * c;
    const u32x2 ks = *reinterpret_cast<const u32x2*>(p.k_scale + so);
    const u32x2 vs = *reinterpret_cast<const u32x2*>(p.v_scale + so);
    pg.ksc = f32x4{f16_bits_to_f32(uint16_t(ks[0])), f16_bits_to_f32(uint16_t(ks[0] >> 16)),
                   f16_bits_to_f32(uint16_t(ks[1])), f16_bits_to_f32(uint16_t(ks[1] >> 16))};
    pg.vsc = f32x4{f16_bits_to_f32(uint16_t(vs[0])), f16_bits_to_f32(uint16_t(vs[0] >> 16)),
                   f16_bits_to_f32(uint16_t(vs[1])), f16_bits_to_f32(uint16_t(vs[1] >> 16))};
  }
}

// V page -> LDS as bf16 [16][D]; logical 16-byte chunk kappa of row rho sits at
// physical chunk kappa ^ (2 * ((rho >> 2) & 3)), so the transposed reads of the
// PV step hit distinct banks.  Rows at or past `valid` are written as zeros.
template <int D>
__device__ __forceinline__ void v_lds_store_chunk(uint16_t* vl, int rho, int kappa, u32x4 w,
                                                  bool zero) {
  constexpr int CPR = D * 2 / 16;
  if (zero) w = u32x4{0u, 0u, 0u, 0u};
  const int phys = kappa ^ (2 * ((rho >> 2) & 3));
  *reinterpret_cast<u32x4*>(vl + rho * D + phys * 8) = w;
  (void)CPR;
}

template <typename KV, int D>
__device__ __forceinline__ void mfma_stage_v(uint16_t* vl, const MfmaPage<KV, D>& pg,
                                             int valid_in_page) {
  const int lane = lane_id();
  if constexpr (sizeof(KV) == 2) {
    constexpr int CPR = D * 2 / 16;                       // bf16 chunks per row
#pragma unroll
    for (int e = 0; e < MfmaPage<KV, D>::VCH; ++e) {
      const int id = lane + kWave * e;
      const int rho = id / CPR, kappa = id % CPR;
      v_lds_store_chunk<D>(vl, rho, kappa, pg.v[e], rho >= valid_in_page);
    }
  } else {
    constexpr int CPR8 = D / 16;                          // int8 chunks per row
#pragma unroll
    for (int e = 0; e < MfmaPage<KV, D>::VCH; ++e) {
      const int id = lane + kWave * e;
      const int rho = id / CPR8, kappa8 = id % CPR8;
      u32x4 lo, hi;
      codes16_to_bf16(pg.v[e], lo, hi);
      v_lds_store_chunk<D>(vl, rho, 2 * kappa8, lo, rho >= valid_in_page);
      v_lds_store_chunk<D>(vl, rho, 2 * kappa8 + 1, hi, rho >= valid_in_page);
    }
  }
}

// A operand of S^T = K Q^T for k-step ks: 8 bf16 of this lane's K row.
template <typename KV, int D>
__device__ __forceinline__ bf16x8 mfma_k_operand(const MfmaPage<KV, D>& pg, int ks) {
  if constexpr (sizeof(KV) == 2) {
    // lane holds D/4 bf16 = KCH 16-byte words; word ks covers d c*D/4 + 8ks .. +8
    return __builtin_bit_cast(bf16x8, pg.k[ks]);
  } else {
    // lane holds D/4 codes; codes 8ks .. 8ks+8 -> bf16
    const u32x4 w = pg.k[ks / 2];
    const int base = (ks & 1) * 2;
    u32x4 r;
    r[0] = codes2_to_bf16x2(w[base], 0);
    r[1] = codes2_to_bf16x2(w[base], 16);
    r[2] = codes2_to_bf16x2(w[base + 1], 0);
    r[3] = codes2_to_bf16x2(w[base + 1], 16);
    return __builtin_bit_cast(bf16x8, r);
  }
}

template <int NRB, int NDB>
struct MfmaState {
  f32x4 acc[NRB][NDB];
  float m[NRB], l[NRB];
};

template <int NRB, int NDB>
__device__ __forceinline__ void mfma_state_store(float* slot, const MfmaState<NRB, NDB>& st) {
  const int lane = lane_id();
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(slot + ((rb * NDB + db) * kWave + lane) * 4) = st.acc[rb][db];
    slot[NRB * NDB * kWave * 4 + rb * kWave + lane] = st.m[rb];
    slot[NRB * NDB * kWave * 4 + (NRB + rb) * kWave + lane] = st.l[rb];
  }
}

template <int NRB, int NDB>
__device__ __forceinline__ void mfma_state_combine(const float* slot, MfmaState<NRB, NDB>& st) {
  const int lane = lane_id();
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float mo = slot[NRB * NDB * kWave * 4 + rb * kWave + lane];
    const float lo = slot[NRB * NDB * kWave * 4 + (NRB + rb) * kWave + lane];
    const float M = fmaxf(st.m[rb], mo);
    const float fa = exp2f(st.m[rb] - M), fb = exp2f(mo - M);
    st.l[rb] = fa * st.l[rb] + fb * lo;
    st.m[rb] = M;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(slot + ((rb * NDB + db) * kWave + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[rb][db][i] = fa * st.acc[rb][db][i] + fb * o[i];
    }
  }
}

template <typename KV, int D, int NRB>
__device__ __forceinline__ void mfma_pass(const AttnParams& p, const Seg& sg, int r0,
                                          uint16_t* vl, float* mrg) {
  constexpr int KS = D / 32;        // 16x16x32 k-steps over d
  constexpr int NDB = D / 16;       // 16-column blocks of d
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, c = lane >> 4;
  const int G = p.G;

  // Q^T operand: lane (l16, c) holds row r0 + 16 rb + l16, d in [c*D/4 + 8ks, +8)
  bf16x8 qB[NRB][KS];
  int lim[NRB];                      // last visible position of the lane's row, -1 if padding
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = r0 + 16 * rb + l16;
    lim[rb] = -1;
    if (r < sg.R) {
      lim[rb] = sg.S + r / G;
      const int64_t qe = out_row(p, sg, r) * D + c * (D / 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qB[rb][ks] = load_q8_bf16(p, qe + 8 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qB[rb][ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }

  MfmaState<NRB, NDB> st;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    st.m[rb] = kNegBig;
    st.l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int valid_end = sg.S + sg.k;
  int j = sg.pa + wave;
  int ids = 0, id_base = j;
  MfmaPage<KV, D> cur, nxt;
  if (j < sg.pe) {
    ids = load_page_ids(p, sg, id_base);
    mfma_load_page<KV, D>(p, readlane(ids, 0), sg.g, cur);
  }
  for (int e = 0; j < sg.pe; j += kWaves, ++e) {
    mfma_stage_v<KV, D>(vl, cur, valid_end - j * kPage);
    const int jn = j + kWaves;
    if (jn < sg.pe) {
      if (e + 1 == kWave) {
        id_base = jn;
        ids = load_page_ids(p, sg, id_base);
        e = -1;
      }
      mfma_load_page<KV, D>(p, readlane(ids, e + 1), sg.g, nxt);
    }
    // ---- scores S^T[token 4c+i][row l16] for every row block
    f32x4 s[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = mfma_k_operand<KV, D>(cur, ks);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[rb][ks], s[rb], 0, 0, 0);
    }
    // ---- online softmax; the lane owns row l16 (+16 rb) and tokens 4c..4c+3
    const int pos0 = j * kPage + 4 * c;
    i16x4 pB[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float sv[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = s[rb][i] * p.scale_log2;
        if constexpr (sizeof(KV) == 1) x *= cur.ksc[i];
        x = (pos0 + i <= lim[rb]) ? x : -INFINITY;
        sv[i] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mn = fmaxf(st.m[rb], mx);
      const float alpha = exp2f(st.m[rb] - mn);
      st.m[rb] = mn;
      float ps = 0.f;
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e2 = exp2f(sv[i] - mn);
        ps += e2;
        float w = e2;
        if constexpr (sizeof(KV) == 1) w = (pos0 + i < valid_end) ? e2 * cur.vsc[i] : 0.f;
        pv[i] = w;
      }
      st.l[rb] = st.l[rb] * alpha + ps;
      const uint32_t lo = pack_bf16x2(pv[0], pv[1]), hi = pack_bf16x2(pv[2], pv[3]);
      pB[rb] = __builtin_bit_cast(i16x4, u32x2{lo, hi});
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[rb][db][i] *= alpha;
      }
    }
    wave_sync();                     // V page visible in LDS
    // ---- O^T[d][row] += V^T[d][tokens] P^T[tokens][row]
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int kappa = 2 * db + (l16 >> 3);
      const int phys = kappa ^ (2 * c);             // rows 4c..4c+3 share the swizzle
      const uint16_t* src = vl + (4 * c) * D + phys * 8 + (l16 & 7);
      const uint32_t v0 = src[0], v1 = src[D], v2 = src[2 * D], v3 = src[3 * D];
      const i16x4 a = __builtin_bit_cast(i16x4, u32x2{v0 | (v1 << 16), v2 | (v3 << 16)});
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        st.acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pB[rb], st.acc[rb][db], 0, 0, 0);
    }
    wave_sync();                     // reads done before the next page overwrites LDS
    cur = nxt;
  }
  // lane partial sums -> row sums (the 4 lanes of a row differ only in c)
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    st.l[rb] += __shfl_xor(st.l[rb], 16, kWave);
    st.l[rb] += __shfl_xor(st.l[rb], 32, kWave);
  }

  // ---- merge the 4 waves: (2,3) -> (0,1) -> 0
  constexpr int SLOT = NRB * NDB * kWave * 4 + 2 * NRB * kWave;
  if (wave >= 2) mfma_state_store<NRB, NDB>(mrg + (wave - 2) * SLOT, st);
  __syncthreads();
  if (wave < 2) mfma_state_combine<NRB, NDB>(mrg + wave * SLOT, st);
  __syncthreads();
  if (wave == 1) mfma_state_store<NRB, NDB>(mrg, st);
  __syncthreads();
  if (wave == 0) {
    mfma_state_combine<NRB, NDB>(mrg, st);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = r0 + 16 * rb + l16;
      if (r >= sg.R) continue;
      if (sg.full) {
        const float inv = 1.f / st.l[rb];
        const int64_t oe = out_row(p, sg, r) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          f32x4 v = st.acc[rb][db];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] *= inv;
          store_out4(p, oe + 16 * db + 4 * c, v);
        }
      } else {
        float* sb = slot_base<D>(p, sg.slot);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          *reinterpret_cast<f32x4*>(sb + int64_t(r) * D + 16 * db + 4 * c) = st.acc[rb][db];
        if (c == 0) {
          sb[int64_t(p.slot_rows) * D + r] = st.m[rb];
          sb[int64_t(p.slot_rows) * (D + 1) + r] = st.l[rb];
        }
      }
    }
  }
  __syncthreads();
}

// ============================================================================
// VALU path
// ============================================================================

template <typename KV, int D>
struct ValuGeom {
  static constexpr int RB = D * int(sizeof(KV));      // bytes per row
  static constexpr int CPR = RB / 16;                 // 16-byte chunks per row
  static constexpr int NCL = kPage * CPR / kWave;     // chunks per lane per page
  static constexpr int QD = D / 4;                    // K values per lane
  static constexpr int CPL = D / 64;                  // output columns per lane
  static constexpr int PAGE_BYTES = kPage * RB;
};

// physical chunk of logical chunk kappa in row rho
template <int CPR>
__device__ __forceinline__ int valu_swz(int rho, int kappa) {
  return kappa ^ (rho & (CPR - 1));
}

template <typename KV, int D>
__device__ __forceinline__ void valu_load_page(const AttnParams& p, int pid, int g, u32x4* kr,
                                               u32x4* vr) {
  using Gm = ValuGeom<KV, D>;
  const int lane = lane_id();
  const int64_t off = page_off<D>(p, pid, g);
  const u32x4* kp = reinterpret_cast<const u32x4*>(static_cast<const KV*>(p.k) + off);
  const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const KV*>(p.v) + off);
#pragma unroll
  for (int e = 0; e < Gm::NCL; ++e) {
    kr[e] = kp[lane + kWave * e];
    vr[e] = vp[lane + kWave * e];
  }
}

template <typename KV, int D>
__device__ __forceinline__ void valu_stage(char* kl, char* vl, const u32x4* kr, const u32x4* vr,
                                           int valid_in_page) {
  using Gm = ValuGeom<KV, D>;
  const int lane = lane_id();
#pragma unroll
  for (int e = 0; e < Gm::NCL; ++e) {
    const int id = lane + kWave * e;
    const int rho = id / Gm::CPR, kappa = id % Gm::CPR;
    const int at = rho * Gm::RB + valu_swz<Gm::CPR>(rho, kappa) * 16;
    *reinterpret_cast<u32x4*>(kl + at) = kr[e];
    *reinterpret_cast<u32x4*>(vl + at) = rho < valid_in_page ? vr[e] : u32x4{0, 0, 0, 0};
  }
}

// decode 16 bytes of KV into floats
template <typename KV>
__device__ __forceinline__ void decode16(u32x4 w, float* f);
template <>
__device__ __forceinline__ void decode16<float>(u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}
template <>
__device__ __forceinline__ void decode16<uint16_t>(u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void decode16<int8_t>(u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int b = 0; b < 4; ++b) f[4 * i + b] = float(int(w[i] << (24 - 8 * b)) >> 24);
  }
}

template <int RV, int CPL>
struct ValuState {
  float o[RV][CPL];
  float m[RV], l[RV];
};

template <int RV, int CPL>
__device__ __forceinline__ void valu_state_store(float* slot, const ValuState<RV, CPL>& st) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < RV; ++r) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) slot[(r * kWave + lane) * CPL + e] = st.o[r][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      slot[RV * kWave * CPL + r] = st.m[r];
      slot[RV * kWave * CPL + RV + r] = st.l[r];
    }
  }
}

template <int RV, int CPL>
__device__ __forceinline__ void valu_state_combine(const float* slot, ValuState<RV, CPL>& st) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    const float mo = slot[RV * kWave * CPL + r];
    const float lo = slot[RV * kWave * CPL + RV + r];
    const float M = fmaxf(st.m[r], mo);
    const float fa = exp2f(st.m[r] - M), fb = exp2f(mo - M);
    st.l[r] = fa * st.l[r] + fb * lo;
    st.m[r] = M;
#pragma unroll
    for (int e = 0; e < CPL; ++e)
      st.o[r][e] = fa * st.o[r][e] + fb * slot[(r * kWave + lane) * CPL + e];
  }
}

// Stage query rows r0 .. r0+RVMAX-1 of the pair into LDS as fp32:
// qs[(r*4 + quarter) * (D/4 + 4) + e]  (the +4 pad spreads quarters over banks)
template <int D>
__device__ __forceinline__ void valu_stage_q(const AttnParams& p, const Seg& sg, int r0,
                                             float* qs) {
  constexpr int QD = D / 4, QP = QD + 4;
  for (int idx = threadIdx.x; idx < kValuRows * D; idx += kAttnThreads) {
    const int r = idx / D, d = idx % D;
    float v = 0.f;
    if (r0 + r < sg.R) {
      const int64_t e = out_row(p, sg, r0 + r) * D + d;
      v = p.q_f32 ? static_cast<const float*>(p.q)[e]
                  : bf16_to_f32(static_cast<const uint16_t*>(p.q)[e]);
    }
    qs[(r * 4 + d / QD) * QP + d % QD] = v;
  }
}

template <typename KV, int D, int RV>
__device__ __forceinline__ void valu_pass(const AttnParams& p, const Seg& sg, int r0, char* wl,
                                          const float* qs, float* mrg) {
  using Gm = ValuGeom<KV, D>;
  constexpr int QD = Gm::QD, QP = QD + 4, CPL = Gm::CPL;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int t = lane & 15, c = lane >> 4;
  char* kl = wl;
  char* vl = wl + Gm::PAGE_BYTES;
  float* ps = reinterpret_cast<float*>(wl + 2 * Gm::PAGE_BYTES);   // [RV][16]
  const int G = p.G;

  ValuState<RV, CPL> st;
  int lim[RV];
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    st.m[r] = kNegBig;
    st.l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) st.o[r][e] = 0.f;
    lim[r] = (r0 + r < sg.R) ? sg.S + (r0 + r) / G : -1;
  }
  const int valid_end = sg.S + sg.k;
  int j = sg.pa + wave;
  int ids = 0;
  u32x4 kr[Gm::NCL], vr[Gm::NCL];
  if (j < sg.pe) {
    ids = load_page_ids(p, sg, j);
    valu_load_page<KV, D>(p, readlane(ids, 0), sg.g, kr, vr);
  }
  for (int e = 0; j < sg.pe; j += kWaves, ++e) {
    const int pid_cur = readlane(ids, e);
    valu_stage<KV, D>(kl, vl, kr, vr, valid_end - j * kPage);
    const int jn = j + kWaves;
    if (jn < sg.pe) {
      if (e + 1 == kWave) {
        ids = load_page_ids(p, sg, jn);
        e = -1;
      }
      valu_load_page<KV, D>(p, readlane(ids, e + 1), sg.g, kr, vr);
    }
    float ksc = 1.f, vsc = 1.f;
    const int pos = j * kPage + t;
    if constexpr (sizeof(KV) == 1) {
      const int64_t so = (int64_t(pid_cur) * p.Hkv + sg.g) * kPage + t;
      ksc = f16_bits_to_f32(p.k_scale[so]);
      vsc = pos < valid_end ? f16_bits_to_f32(p.v_scale[so]) : 0.f;
    }
    wave_sync();
    // ---- this lane's quarter of K row t as fp32
    float kf[QD];
    constexpr int CQ = Gm::CPR / 4;            // chunks per quarter
    constexpr int FPC = 16 / int(sizeof(KV));  // floats per chunk
#pragma unroll
    for (int e2 = 0; e2 < CQ; ++e2) {
      const int kappa = c * CQ + e2;
      const u32x4 w = *reinterpret_cast<const u32x4*>(kl + t * Gm::RB + valu_swz<Gm::CPR>(t, kappa) * 16);
      decode16<KV>(w, kf + e2 * FPC);
    }
    float s[RV];
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const float* qrow = qs + (r * 4 + c) * QP;
      float a = 0.f;
#pragma unroll
      for (int e4 = 0; e4 < QD / 4; ++e4) {
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(qrow + 4 * e4);
        a = fmaf(q4[0], kf[4 * e4], a);
        a = fmaf(q4[1], kf[4 * e4 + 1], a);
        a = fmaf(q4[2], kf[4 * e4 + 2], a);
        a = fmaf(q4[3], kf[4 * e4 + 3], a);
      }
      a += __shfl_xor(a, 16, kWave);
      a += __shfl_xor(a, 32, kWave);
      s[r] = a;
    }
    // ---- online softmax over the 16 tokens of the page (16-lane groups);
    //      the running output is rescaled as soon as a row's maximum moves
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const float x = (pos <= lim[r]) ? s[r] * p.scale_log2 * ksc : -INFINITY;
      const float mx = group_max<16>(x);
      const float mn = fmaxf(st.m[r], mx);
      const float alpha = exp2f(st.m[r] - mn);
      st.m[r] = mn;
      const float e2 = exp2f(x - mn);
      st.l[r] = st.l[r] * alpha + e2;
#pragma unroll
      for (int e3 = 0; e3 < CPL; ++e3) st.o[r][e3] *= alpha;
      if (c == 0) ps[r * kPage + t] = e2 * vsc;
    }
    wave_sync();
    // ---- O[r][cols] += sum_t p[r][t] V[t][cols], four tokens at a time
    const int cb = lane * CPL * int(sizeof(KV));   // byte of this lane's first column
    const int kappa_v = cb / 16, within = cb % 16;
#pragma unroll
    for (int t0 = 0; t0 < kPage; t0 += 4) {
      float vv[4][CPL];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int row = t0 + tt;
        const char* src = vl + row * Gm::RB + valu_swz<Gm::CPR>(row, kappa_v) * 16 + within;
        if constexpr (sizeof(KV) == 4) {
#pragma unroll
          for (int e2 = 0; e2 < CPL; ++e2) vv[tt][e2] = reinterpret_cast<const float*>(src)[e2];
        } else if constexpr (sizeof(KV) == 2) {
          if constexpr (CPL == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
            vv[tt][0] = bf16_lo(w);
            vv[tt][CPL - 1] = bf16_hi(w);
          } else {
            vv[tt][0] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(src));
          }
        } else {
#pragma unroll
          for (int e2 = 0; e2 < CPL; ++e2)
            vv[tt][e2] = float(reinterpret_cast<const int8_t*>(src)[e2]);
        }
      }
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        const f32x4 pw = *reinterpret_cast<const f32x4*>(ps + r * kPage + t0);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
          for (int e2 = 0; e2 < CPL; ++e2) st.o[r][e2] = fmaf(pw[tt], vv[tt][e2], st.o[r][e2]);
        }
      }
    }
    wave_sync();
  }
#pragma unroll
  for (int r = 0; r < RV; ++r) st.l[r] = group_sum<16>(st.l[r]);

  constexpr int SLOT = RV * kWave * CPL + 2 * RV;
  if (wave >= 2) valu_state_store<RV, CPL>(mrg + (wave - 2) * SLOT, st);
  __syncthreads();
  if (wave < 2) valu_state_combine<RV, CPL>(mrg + wave * SLOT, st);
  __syncthreads();
  if (wave == 1) valu_state_store<RV, CPL>(mrg, st);
  __syncthreads();
  if (wave == 0) {
    valu_state_combine<RV, CPL>(mrg, st);
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const int rr = r0 + r;
      if (rr >= sg.R) continue;
      if (sg.full) {
        const float inv = 1.f / st.l[r];
        const int64_t oe = out_row(p, sg, rr) * D + lane * CPL;
#pragma unroll
        for (int e2 = 0; e2 < CPL; ++e2) store_out1(p, oe + e2, st.o[r][e2] * inv);
      } else {
        float* sb = slot_base<D>(p, sg.slot);
#pragma unroll
        for (int e2 = 0; e2 < CPL; ++e2) sb[int64_t(rr) * D + lane * CPL + e2] = st.o[r][e2];
        if (lane == 0) {
          sb[int64_t(p.slot_rows) * D + rr] = st.m[r];
          sb[int64_t(p.slot_rows) * (D + 1) + rr] = st.l[r];
        }
      }
    }
  }
  __syncthreads();
}

// ============================================================================
// cross-workgroup merge of a pair split over several workgroups
// ============================================================================

__device__ __forceinline__ int64_t range_start(int w, int64_t N, int W) {
  return int64_t(w) * N / W;
}
// the workgroup (logical index) whose range holds global page x
__device__ __forceinline__ int wg_of(int64_t x, int64_t N, int W) {
  return int(((x + 1) * W - 1) / N);
}
__device__ __forceinline__ int slot_of(int w, int64_t pair_begin, int64_t N, int W) {
  const int64_t s = range_start(w, N, W);
  return (max(s, pair_begin) == s) ? 2 * w : 2 * w + 1;
}

template <int D>
__device__ void merge_pair(const AttnParams& p, const Seg& sg, int64_t pb, int64_t pend,
                           int64_t N) {
  const int wf = wg_of(pb, N, p.W), wl = wg_of(pend - 1, N, p.W);
  const int items = sg.R * (D / 4);
  for (int it = threadIdx.x; it < items; it += kAttnThreads) {
    const int r = it / (D / 4), d4 = it % (D / 4);
    float M = kNegBig, L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    for (int w = wf; w <= wl; ++w) {
      if (range_start(w + 1, N, p.W) == range_start(w, N, p.W)) continue;   // empty range
      const float* sb = slot_base<D>(p, slot_of(w, pb, N, p.W));
      const float ms = sb[int64_t(p.slot_rows) * D + r];
      const float ls = sb[int64_t(p.slot_rows) * (D + 1) + r];
      const f32x4 os = *reinterpret_cast<const f32x4*>(sb + int64_t(r) * D + 4 * d4);
      const float Mn = fmaxf(M, ms);
      const float fa = exp2f(M - Mn), fb = exp2f(ms - Mn);
      L = fa * L + fb * ls;
#pragma unroll
      for (int i = 0; i < 4; ++i) O[i] = fa * O[i] + fb * os[i];
      M = Mn;
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int i = 0; i < 4; ++i) O[i] *= inv;
    store_out4(p, out_row(p, sg, r) * D + 4 * d4, O);
  }
}

// ============================================================================
// kernel
// ============================================================================

template <typename KV, int D>
struct AttnLds {
  using Gm = ValuGeom<KV, D>;
  static constexpr int VALU_WAVE = 2 * Gm::PAGE_BYTES + kValuRows * kPage * 4;
  static constexpr int MFMA_WAVE = kPage * D * 2;
  static constexpr int WAVE = VALU_WAVE > MFMA_WAVE ? VALU_WAVE : MFMA_WAVE;
  static constexpr int QS = kValuRows * 4 * (D / 4 + 4);
  static constexpr int MERGE_MFMA = 2 * (D / 16) * kWave * 4 + 4 * kWave;
  static constexpr int MERGE_VALU = kValuRows * kWave * (D / 64) + 2 * kValuRows;
  static constexpr int MERGE = 2 * (MERGE_MFMA > MERGE_VALU ? MERGE_MFMA : MERGE_VALU);
};

template <typename KV, int D>
__device__ __forceinline__ void process_segment(const AttnParams& p, const Seg& sg, char* wl,
                                                float* qs, float* mrg) {
  bool use_mfma = false;
  if constexpr (sizeof(KV) != 4) use_mfma = p.path == 2 || (p.path == 0 && sg.R >= 16);
  if constexpr (sizeof(KV) != 4) {
    if (use_mfma) {
      for (int r0 = 0; r0 < sg.R; r0 += kMfmaRows) {
        if (sg.R - r0 > 16)
          mfma_pass<KV, D, 2>(p, sg, r0, reinterpret_cast<uint16_t*>(wl), mrg);
        else
          mfma_pass<KV, D, 1>(p, sg, r0, reinterpret_cast<uint16_t*>(wl), mrg);
      }
      return;
    }
  }
  for (int r0 = 0; r0 < sg.R; r0 += kValuRows) {
    valu_stage_q<D>(p, sg, r0, qs);
    __syncthreads();
    const int rn = sg.R - r0;
    if (rn <= 4) valu_pass<KV, D, 4>(p, sg, r0, wl, qs, mrg);
    else if (rn <= 8) valu_pass<KV, D, 8>(p, sg, r0, wl, qs, mrg);
    else valu_pass<KV, D, 16>(p, sg, r0, wl, qs, mrg);
  }
}

template <typename KV, int D>
__global__ __launch_bounds__(kAttnThreads, 1) void verify_attn_kernel(AttnParams p) {
  using L = AttnLds<KV, D>;
  __shared__ int32_t s_start[kMaxB + 1];
  __shared__ int32_t s_wtot[kWaves];
  __shared__ int s_flag;
  __shared__ __attribute__((aligned(16))) char s_wave[kWaves * L::WAVE];
  __shared__ __attribute__((aligned(16))) float s_q[L::QS];
  __shared__ __attribute__((aligned(16))) float s_mrg[L::MERGE];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;

  // ---- exclusive prefix over sequences of Hkv * pages
  const int B = p.B;
  const int per = (B + kAttnThreads - 1) / kAttnThreads;
  int tot = 0;
  for (int e = 0; e < per; ++e) {
    const int b = tid * per + e;
    if (b < B) tot += p.Hkv * seq_info(p, b).np;
  }
  int incl = tot;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) s_wtot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wtot[w];
  int run = base + incl - tot;
  for (int e = 0; e < per; ++e) {
    const int b = tid * per + e;
    if (b < B) {
      s_start[b] = run;
      run += p.Hkv * seq_info(p, b).np;
    }
  }
  if (tid == kAttnThreads - 1) s_start[B] = base + incl;
  __syncthreads();
  const int64_t N = s_start[B];
  if (N == 0) return;

  // ---- this workgroup's page range; consecutive ranges go to one XCD
  const int h = blockIdx.x;
  const int w = (p.W % 8 == 0) ? (h % 8) * (p.W / 8) + h / 8 : h;
  const int64_t g0 = range_start(w, N, p.W), g1 = range_start(w + 1, N, p.W);
  if (g0 >= g1) return;

  int b = 0;
  {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= g0) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  char* wl = s_wave + wave * L::WAVE;
  int64_t cur = g0;
  while (cur < g1) {
    while (b < B - 1 && s_start[b + 1] <= cur) ++b;
    const SeqInfo si = seq_info(p, b);
    const int64_t sb = s_start[b];
    const int o = int(cur - sb);
    Seg sg;
    sg.b = b;
    sg.g = o / si.np;
    sg.pa = o - sg.g * si.np;
    sg.S = si.S;
    sg.k = si.k;
    sg.q0 = si.q0;
    sg.np = si.np;
    sg.R = si.k * p.G;
    const int64_t pb = sb + int64_t(sg.g) * si.np;
    const int64_t pend = pb + si.np;
    const int64_t se = min(g1, pend);
    sg.pe = int(se - pb);
    sg.full = (cur == pb) && (se == pend);
    sg.slot = (cur == g0) ? 2 * w : 2 * w + 1;

    process_segment<KV, D>(p, sg, wl, s_q, s_mrg);

    if (!sg.full) {
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        const int wf = wg_of(pb, N, p.W), wlast = wg_of(pend - 1, N, p.W);
        int nseg = 0;
        for (int x = wf; x <= wlast; ++x)
          nseg += range_start(x + 1, N, p.W) > range_start(x, N, p.W);
        const int old = atomicAdd(p.counters + wf, 1);
        s_flag = (old == nseg - 1);
      }
      __syncthreads();
      if (s_flag) {
        __threadfence();
        merge_pair<D>(p, sg, pb, pend, N);
        if (tid == 0) atomicExch(p.counters + wg_of(pb, N, p.W), 0);
      }
      __syncthreads();
    }
    cur = se;
  }
}

// ============================================================================
// host side
// ============================================================================

AttnPlan plan_verify_attn(const sva_batch* batch, const sva_paged_kv* kv, int Hq, int num_cus,
                          const sva_verify_opts* opts) {
  AttnPlan pl;
  const int G = Hq / kv->Hkv;
  const int64_t pages_per_seq =
      std::min<int64_t>(kv->max_pages_per_seq, (int64_t(batch->max_len) + kPage - 1) / kPage);
  const int64_t pages_ub = int64_t(batch->B) * kv->Hkv * std::max<int64_t>(pages_per_seq, 1);
  int W = 0;
  if (opts && opts->num_workgroups > 0) {
    W = opts->num_workgroups;
  } else {
    const int64_t want = (pages_ub + 15) / 16;     // at least 4 pages per wave
    W = int(std::min<int64_t>(std::max(num_cus, 1), std::max<int64_t>(want, 1)));
  }
  pl.num_wg = W;
  pl.slot_rows = std::max(batch->max_q, 1) * G;
  pl.counter_bytes = (size_t(W) * 4 + 255) & ~size_t(255);
  pl.slot_bytes = size_t(2) * W * pl.slot_rows * (kv->d + 2) * sizeof(float);
  pl.total_bytes = pl.counter_bytes + pl.slot_bytes;
  return pl;
}

template <typename KV, int D>
static hipError_t attn_launch(const AttnParams& p, hipStream_t st) {
  hipLaunchKernelGGL((verify_attn_kernel<KV, D>), dim3(p.W), dim3(kAttnThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_verify_attn(const sva_batch* batch, const void* q, int q_dtype, int Hq,
                              const sva_paged_kv* kv, float softmax_scale, void* out,
                              int out_dtype, int path, const AttnPlan& plan, void* workspace,
                              hipStream_t st) {
  AttnParams p;
  p.q = q;
  p.k = kv->k;
  p.v = kv->v;
  p.k_scale = static_cast<const uint16_t*>(kv->k_scale);
  p.v_scale = static_cast<const uint16_t*>(kv->v_scale);
  p.block_table = kv->block_table;
  p.ctx_lens = batch->ctx_lens;
  p.cu_q = batch->cu_q;
  p.out = out;
  p.counters = static_cast<int32_t*>(workspace);
  p.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.counter_bytes);
  p.scale_log2 = softmax_scale * kLog2e;
  p.q_f32 = q_dtype == SVA_F32;
  p.out_f32 = out_dtype == SVA_F32;
  p.B = batch->B;
  p.T = batch->total_q;
  p.Hq = Hq;
  p.Hkv = kv->Hkv;
  p.G = Hq / kv->Hkv;
  p.num_pages = kv->num_pages;
  p.max_pages = kv->max_pages_per_seq;
  p.max_q = batch->max_q;
  p.slot_rows = plan.slot_rows;
  p.W = plan.num_wg;
  p.path = path;
  if (kv->kv_dtype == SVA_F32)
    return kv->d == 64 ? attn_launch<float, 64>(p, st) : attn_launch<float, 128>(p, st);
  if (kv->kv_dtype == SVA_BF16)
    return kv->d == 64 ? attn_launch<uint16_t, 64>(p, st) : attn_launch<uint16_t, 128>(p, st);
  return kv->d == 64 ? attn_launch<int8_t, 64>(p, st) : attn_launch<int8_t, 128>(p, st);
}

}  // namespace sva
