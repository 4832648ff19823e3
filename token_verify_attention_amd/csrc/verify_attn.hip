// Causal multi-query verification attention over a paged KV cache, gfx950.
//
// What is computed ("Decoding Speculative Decoding from First Principles",
// section "Speculating to get sequence parallelism during decode"; "CXL-SpecKV",
// key observation (1)): for sequence b, draft query i and query head h (kv head
// g = h / G), softmax(scale * q . K_p) V_p over positions p = 0 .. S_b + i.
// Split-KV with an online softmax reaches exactly that result; every partial
// carries (running max m, weight sum l, unnormalised output O), maxima in the
// log2 domain (scores pre-multiplied by scale * log2 e, exp2 throughout).
//
// Work decomposition.  The pages of all (sequence, kv-head) pairs are laid end
// to end; workgroup w streams the contiguous range [w*N/W, (w+1)*N/W) of that
// list, which may cover the tail of one pair, whole pairs and the head of
// another, so every workgroup moves the same number of pages.  Each (b, g)
// segment is shared by the 4 waves of the workgroup, each taking every 4th
// pair of consecutive pages, so the k_b*G query rows of the pair share every
// K/V page load (one KV read amortised over all drafts and the GQA group:
// "Decoding Speculative Decoding...", sequence-parallel section).  Waves merge
// through LDS; a pair that spans several workgroups leaves partials in the
// workspace and the last workgroup to finish it (device-scope counter) merges
// them, so the whole call is one kernel.
//
// Memory pipeline.  Each wave owns a ring of LDS page slots filled by
// global_load_lds_dwordx4 (HBM -> LDS without registers, 1 KB per wave
// instruction, 16-byte chunks permuted per row so later LDS reads are free of
// bank conflicts).  Steps of 2 pages are issued S steps ahead and waited for
// with explicit vmcnt counts; page ids come from scalar loads.
//
// Inner loops per step (32 tokens):
//  * MFMA path (bf16 and INT8 caches, any k_b*G; blocks of 16 query rows are
//    padded, which costs nothing while the loop is HBM-bound): S^T = K Q^T
//    with v_mfma_f32_16x16x32_bf16 (a lane owns one query row and 4 tokens of
//    a page), O^T += V^T P^T with v_mfma_f32_16x16x16_bf16.  INT8 per-token
//    scales multiply the score (K) and the probability (V).
//  * VALU path (fp32 caches; bf16 / INT8 on request): lane = (token, half of
//    d); bf16 dot2 products (INT8 codes convert exactly to bf16), online
//    softmax over 32-lane groups, P.V with bf16 probability pairs and dot2,
//    each lane owning d/64 columns.  fp32 caches use plain fp32 FMAs.
//
// Positions at or past S_b + k_b (garbage slots of the last page) are masked
// in the scores and zeroed in V, so NaN garbage never reaches an output.
#include "common.h"
#include "launch.h"
#include "kv_rows.h"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace sva {

// Waves per workgroup: the INT8 MFMA kernel runs 8 (two per SIMD, so one
// wave's LDS, conversion and MFMA latencies hide behind the other's work; its
// pages are small enough for two ring steps per wave), the others 4 (bf16
// pages fill the ring with 4 waves x 2 steps; the VALU kernels' register use
// allows one wave per SIMD only).
constexpr int kWavesInt8 = 8;
constexpr int kWavesValu = 4;
// The workspace starts with two completion counters per possible workgroup
// (arrivals, publications), at a fixed size, so partial slots of one call never
// overlap the counters of a later call with a different grid.
constexpr int kMaxWorkgroups = 4096;
constexpr int kMfmaRows = 32;
constexpr int kValuRows = 16;
constexpr int kMaxDraftsSplit = 16;            // max_q the split kernel takes
constexpr int kMaxRowsSplit = 128;             // max_q * G the split kernel takes
constexpr int kRingBudget = 136 * 1024;        // LDS bytes for the page rings of all waves
constexpr float kNegBig = -1.0e30f;            // finite start value of running maxima
// Streaming time a segment's fixed work costs (its query rows, first copies
// and merge), as bytes of KV: the work split counts it once per segment.
constexpr int kSegCostBytes = 96 * 1024;
constexpr float kLog2e = 1.4426950408889634f;

#define AS1 __attribute__((address_space(1)))
#define AS3 __attribute__((address_space(3)))
#define AS4 __attribute__((address_space(4)))

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* cu_q;
  const uint32_t* draft_mask;   // [T] tree attention masks, or NULL (causal drafts)
  const void* k_new;            // [T, Hkv, d] new rows to append first, or NULL
  const void* v_new;
  int src_f32;                  // element type of k_new / v_new: fp32, else bf16
  void* out;
  float* partials;
  int32_t* counters;
  int32_t* status;      // workspace status word: bit 0 set when a split-pair wait gave up
  int wait_polls;       // bound on the polls of that wait
  float scale_log2;     // softmax_scale * log2(e)
  int q_f32, out_f32;
  int B, T, Hq, Hkv, G, num_pages, max_pages, max_q;
  int slot_rows;        // rows per partial slot (max_q * G)
  int W;                // grid size
  int seg_cost;         // fixed cost of a segment, in pages (work split)
  // Pairs are (sequence, g) with kv head g >> kv_shift: the G query heads of
  // a kv head form 2^kv_shift pairs (Hkv and G above count those pairs),
  // streamed by different workgroups.
  int kv_shift;
  // Row-block kernel: key slices per row block (1: each block streams all of
  // its pair's pages and writes its rows; more: each slice writes partial
  // states that a second launch merges).
  int rows_nseg;
};

struct SeqInfo {
  int S, k, q0, np;
};

// Keys a query row sees: the committed context 0 .. S-1 and some drafts, kept
// in one register per row.  Mask form: bit j set when draft j is visible --
// the caller's tree mask, or bits 0 .. i for causal draft i (at most 32
// drafts).  Index form (causal calls of the row-block kernel, up to 1024
// drafts): the draft index i, drafts 0 .. i visible.  The draft range end
// S + k is the segment's; padding rows see no draft.
__device__ __forceinline__ uint32_t row_mask(const AttnParams& p, int q0, int i) {
  return p.draft_mask ? p.draft_mask[q0 + i] : (2u << i) - 1u;
}
__device__ __forceinline__ bool key_visible(int pos, int S, int end, uint32_t mask) {
  return pos < S || (pos < end && ((mask >> ((pos - S) & 31)) & 1u));
}
__device__ __forceinline__ bool key_visible_idx(int pos, int S, int end, int i) {
  return pos < S || (pos < end && pos - S <= i);
}

// Sequence b with every device-resident value clamped into the buffers.
// The three loads are independent and the page count is computed without a
// branch, so one memory round trip serves them all.
__device__ __forceinline__ SeqInfo seq_info(const AttnParams& p, int b) {
  const int c0 = p.cu_q[b], c1 = p.cu_q[b + 1], ctx = p.ctx_lens[b];
  const int q0 = min(max(c0, 0), p.T);
  const int q1 = min(max(c1, q0), p.T);
  SeqInfo s;
  s.q0 = q0;
  s.k = min(q1 - q0, p.max_q);
  s.S = max(ctx, 0);
  const int64_t need = (int64_t(s.S) + s.k + kPage - 1) / kPage;
  s.np = s.k > 0 ? int(min(need, int64_t(p.max_pages))) : 0;
  return s;
}

// The work split runs in cost coordinates: the Hkv pairs of sequence b lie
// end to end from the sequence's start sb, each taking seg_cost + np units --
// its np pages between seg_cost / 2 virtual units before and the rest after
// (the fixed cost of a segment: its query rows, first copies and merge, half
// at either end so that a pair split in two costs its halves alike) -- and
// every workgroup takes an equal contiguous range of the total.  A range of
// many short pairs thus holds fewer pages than a range inside one long pair,
// and a batch of equal pairs is split exactly as by pages alone.
__device__ __forceinline__ int64_t seq_cost(const AttnParams& p, const SeqInfo& si) {
  return si.np > 0 ? int64_t(p.Hkv) * (si.np + p.seg_cost) : 0;
}
struct PairPos {
  int g;              // kv head
  int pa, pe;         // pages of the pair inside [cur, c1) (empty when pe <= pa)
  int64_t pb, pend;   // cost coordinates of the pair's first page and past its last
  int64_t bend;       // end of the pair's block (the next pair's start)
};
__device__ __forceinline__ PairPos pair_pos(const AttnParams& p, int64_t cur, int64_t sb,
                                            int np, int64_t c1) {
  const int blk = np + p.seg_cost;
  PairPos r;
  r.g = int(cur - sb) / blk;
  r.pb = sb + int64_t(r.g) * blk + p.seg_cost / 2;
  r.pend = r.pb + np;
  r.bend = sb + int64_t(r.g + 1) * blk;
  r.pa = int(max(cur, r.pb) - r.pb);
  r.pe = int(max(min(c1, r.pend), r.pb) - r.pb);
  return r;
}

struct Seg {
  int b, g, S, k, q0, np;
  int pa, pe;     // page range within the pair
  int R;          // query rows of the pair: k * G
  bool full;      // the segment is the whole pair
  int slot;       // partial slot when !full
  bool fuse;      // split pair merged with the last workgroup's wave merge
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The thread index for the merges after the page loop.  Pinned (through a
// volatile move), the merge's index math is not hoisted out of the segment
// loop, where it would hold registers through the page loop: the INT8 kernel
// (256 VGPRs for 8 waves) would spill, and in the bf16 kernel the hoisted
// cross-workgroup merge measurably slows the page loop.  The wave merge of
// the bf16 kernel keeps the hoisted (precomputed) form, which takes its index
// math off the path after the last page.
// Row factors of the wave merge: kMergeTab floats per query row (up to 32
// rows): the weights of up to 8 waves, then the maximum and the denominator.
constexpr int kMergeTab = 12;
__device__ __forceinline__ float* merge_table() {
  __shared__ __attribute__((aligned(16))) float s_tab[32 * kMergeTab];
  return s_tab;
}

template <bool kPin>
__device__ __forceinline__ int merge_tid() {
  int tid = int(threadIdx.x);
  if constexpr (kPin) asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(tid));
  return tid;
}

// This thread's wave within the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
}

__device__ __forceinline__ int clamp_page(int pid, int num_pages) {
  return min(max(pid, 0), num_pages - 1);
}

// Physical page of logical page j of sequence b (a wave-uniform scalar load).
__device__ __forceinline__ int page_id(const AttnParams& p, int b, int j) {
  const AS4 int32_t* bt = (const AS4 int32_t*)p.block_table;
  return clamp_page(bt[int64_t(b) * p.max_pages + j], p.num_pages);
}

// ---- output and partial-slot addressing -----------------------------------

__device__ __forceinline__ int64_t out_row(const AttnParams& p, const Seg& sg, int r) {
  const int i = r / p.G;
  const int j = r - i * p.G;
  return (int64_t(sg.q0 + i) * p.Hq + sg.g * p.G + j);
}

template <int D>
__device__ __forceinline__ float* slot_base(const AttnParams& p, int slot) {
  return p.partials + int64_t(slot) * p.slot_rows * (D + 2);
}

// Partial slots and completion counters are shared by workgroups that may sit
// on different XCDs, each with its own L2.  They are accessed with device-scope
// relaxed atomics (sc1 loads and stores, coherent across XCDs), so no fence has
// to write back or invalidate a whole L2: an s_waitcnt on the writer's stores
// before the counter increment orders them.
__device__ __forceinline__ void st_dev(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte variants through a buffer resource over one partial slot: the same
// sc1 (device-coherent) policy in one instruction instead of four.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kCpolSc1);
}
__device__ __forceinline__ f32x4 ld_dev4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCpolSc1);
}
// 4-byte device-coherent load that is not an atomic: the compiler keeps many
// in flight (it waits after every atomic load).
__device__ __forceinline__ float ld_dev1(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCpolSc1));
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
// page ring: geometry, DMA and waits
// ============================================================================

template <typename KV, int D, int NW>
struct Geo {
  static constexpr int ES = int(sizeof(KV));
  static constexpr int RB = D * ES;                  // bytes per K (or V) row
  static constexpr int CPR = RB / 16;                // 16-byte chunks per row
  static constexpr int PAGE = kPage * RB;            // bytes of one page of one head
  static constexpr int SCALES = ES == 1 ? 64 : 0;    // INT8: 16 K + 16 V fp16 scales
  static constexpr int SLOT = 2 * PAGE + SCALES;     // one ring slot: K page, V page, scales
  static constexpr int DMA = PAGE / 1024;            // dwordx4 DMA instructions per page half
  static constexpr int P = 2 * DMA + (ES == 1 ? 1 : 0);   // DMA instructions per page
  static constexpr int S_RAW = kRingBudget / (NW * 2 * SLOT);
  static constexpr int S = S_RAW < 1 ? 1 : (S_RAW > 3 ? 3 : S_RAW);   // steps held in the ring
  static constexpr int RING = 2 * S * SLOT;          // bytes per wave

  // 16-byte chunks are permuted inside each row (XOR of the chunk index) so
  // that the LDS reads of a 16-lane group hit distinct banks (a 256-byte bank
  // window holds RPW rows).
  static constexpr int RPW = RB >= 256 ? 1 : 256 / RB;
  // K: 16 lanes read one chunk (or half chunk) of 16 consecutive rows.  Rows
  // of 256 bytes or more XOR the chunk with the row's two 2-bit halves
  // swapped: with the plain row index (rows 0-3 reading chunks 0-3, ...), a
  // 16-byte read of the MFMA operand layout measured 4 bank-conflict cycles
  // per instruction on gfx950 (126 bytes per clock per CU); with the halves
  // swapped, none (187 bytes per clock).
  static __device__ __forceinline__ int swz_k(int rho) {
    return RB >= 256 ? (((rho & 3) << 2) | ((rho >> 2) & 3)) & (CPR - 1) : (rho / RPW) & (CPR - 1);
  }
  // V: bf16 -- 4 rows x 32 contiguous bytes (transposing 16-bit reads);
  // INT8 -- 4 rows x 16 bytes of each of 2 pages (transposing 8-bit reads);
  // fp32 -- 4-row quads (VALU path).  The 16-lane groups of rows 4c .. 4c+3
  // and 4c+4 .. 4c+7 read together, so bit 2 of the row also moves the
  // chunks (bf16: by half a bank window; INT8: into the slots the other
  // group leaves free); without it the two groups hit the same banks
  // (measured: bank-conflict cycles 2.3-2.7x the LDS-active cycles, halved
  // by this term).
  static __device__ __forceinline__ int swz_v(int rho) {
    return ES == 4 ? ((rho >> 2) & 3) * 2
                   : (ES == 2 ? (2 * (rho & 3)) ^ ((RB >= 256 ? 8 : 2) * ((rho >> 2) & 1))
                              : ((rho & 3) ^ (RB >= 128 ? (rho >> 2) & 1 : 0)));
  }
};

// Global -> LDS copies (lane l's 16 or 4 bytes land at l * 16 or l * 4 past
// the wave-uniform LDS address in M0).  Issued through asm on purpose: for
// the builtin, this compiler makes every later LDS read wait for all DMAs in
// flight (vmcnt(0)), which would drain the ring at each step.  The ring's own
// waits (wait_steps) order these copies against the reads; M0 is written
// here, and one wait state separates the write from its use.  KV pages are
// read exactly once per call, so the loads carry the non-temporal hint
// (streamed through the caches): measured 6.6-6.7 TB/s for this ring against
// 5.9 TB/s without it.
__device__ __forceinline__ uint32_t lds_addr(const void* l) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((AS3 const void*)l));
}
// The global address is a wave-uniform base in SGPRs plus a 32-bit per-lane
// offset (the saddr form), so issuing a page costs no 64-bit vector adds.
// kNT = false (the row-block kernel: several workgroups read each page) drops
// the non-temporal hint so the pages stay in L2 for the other readers.
template <bool kNT = true>
__device__ __forceinline__ void dma16(const void* base, uint32_t off, void* l) {
  if constexpr (kNT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 ::"v"(off), "s"(base), "s"(lds_addr(l)) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 ::"v"(off), "s"(base), "s"(lds_addr(l)) : "memory", "m0");
}
// 4 bytes per lane from a per-lane 64-bit address (lanes may read different
// arrays).
template <bool kNT = true>
__device__ __forceinline__ void dma4(const void* src, void* l) {
  if constexpr (kNT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt"
                 ::"v"(src), "s"(lds_addr(l)) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 ::"v"(src), "s"(lds_addr(l)) : "memory", "m0");
}

// Page `pid` of kv head g -> ring slot (K page, V page, INT8 scales).
template <typename KV, int D, bool kNT = true>
__device__ __forceinline__ void dma_page(const AttnParams& p, int pid, int g, char* slot) {
  using Gm = Geo<KV, D, kWavesValu>;      // page geometry only
  const int lane = lane_id();
  const int64_t off = (int64_t(pid) * (p.Hkv >> p.kv_shift) + (g >> p.kv_shift)) * Gm::PAGE;
  const char* kb = static_cast<const char*>(p.k) + off;
  const char* vb = static_cast<const char*>(p.v) + off;
#pragma unroll
  for (int e = 0; e < Gm::DMA; ++e) {
    const int phys = kWave * e + lane;
    const int rho = phys / Gm::CPR, phi = phys % Gm::CPR;
    dma16<kNT>(kb, uint32_t(rho * Gm::RB + (phi ^ Gm::swz_k(rho)) * 16), slot + 1024 * e);
    dma16<kNT>(vb, uint32_t(rho * Gm::RB + (phi ^ Gm::swz_v(rho)) * 16),
               slot + Gm::PAGE + 1024 * e);
  }
  if constexpr (Gm::ES == 1) {
    // one copy for both scale rows: lanes 0-7 the 16 K scales, lanes 8-15
    // the 16 V scales, landing side by side
    const int64_t so = (int64_t(pid) * (p.Hkv >> p.kv_shift) + (g >> p.kv_shift)) * kPage;
    if (lane < 16)
      dma4<kNT>((lane < 8 ? p.k_scale : p.v_scale) + so + 2 * (lane & 7), slot + 2 * Gm::PAGE);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most `pending` later steps (P2 DMA instructions each) are in flight.
template <int P2, int S>
__device__ __forceinline__ void wait_steps(int pending) {
  if constexpr (S >= 3) {
    if (pending >= 2) { wait_vm<2 * P2>(); return; }
  }
  if constexpr (S >= 2) {
    if (pending >= 1) { wait_vm<P2>(); return; }
  }
  wait_vm<0>();
}

// Streams this wave's pages of the segment through its ring and calls
// st.step(slot of page a, slot of page a+1, a, page a+1 exists) for each pair
// of consecutive pages (a = pa + 2u, u = wave, wave + 4, ...).
template <typename KV, int D, int NW>
__device__ __forceinline__ void issue_step(const AttnParams& p, const Seg& sg, char* ring, int wave,
                                           int s) {
  using Gm = Geo<KV, D, NW>;
  const int a = sg.pa + 2 * (wave + NW * s);
  // both ids with in-range indices and no branch: the loads go out together
  // (past the segment's end the second slot gets a copy of the first page)
  const int ida = page_id(p, sg.b, a);
  const int idb = page_id(p, sg.b, min(a + 1, sg.pe - 1));
  char* slots = ring + (s % Gm::S) * 2 * Gm::SLOT;
  dma_page<KV, D>(p, ida, sg.g, slots);
  dma_page<KV, D>(p, idb, sg.g, slots + Gm::SLOT);
}

// The first steps of a wave's share of a segment: every page id is loaded
// before the first copy is issued, so the prologue costs one memory round
// trip for its ids instead of one per page.
template <typename KV, int D, int NW, int S>
__device__ __forceinline__ void issue_first_steps(const AttnParams& p, const Seg& sg, char* ring,
                                                  int wave, const int (&q)[S]) {
  using Gm = Geo<KV, D, NW>;
  int ids[S][2];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int a = min(sg.pa + 2 * (wave + NW * i), sg.pe - 1);
    ids[i][0] = page_id(p, sg.b, a);
    ids[i][1] = page_id(p, sg.b, min(a + 1, sg.pe - 1));
  }
#pragma unroll
  for (int i = 0; i < S; ++i) {
    if (q[i] < 0) continue;
    char* slots = ring + (i % Gm::S) * 2 * Gm::SLOT;
    dma_page<KV, D>(p, ids[i][0], sg.g, slots);
    dma_page<KV, D>(p, ids[i][1], sg.g, slots + Gm::SLOT);
  }
}

// Steps of a step type that separates its LDS reads (load) from its arithmetic
// (compute).  Wave w takes units (pairs of pages) w, w + NW, w + 2 NW, ... of
// the segment -- a fixed assignment, so results are reproducible bit for bit.
// q[0 .. S-1] are the units this wave has in flight, oldest first (-1: none);
// q[0] is processed.  Once the step's reads have landed, its slot is free and
// the copy of unit q[0] + NW * S into it is issued before the softmax and P.V
// work, so it has that work's time to arrive.  EDGE = false runs while q[0] is
// at most ulim (steps that need no masks) and EDGE = true runs the rest.
template <typename KV, int D, int NW, bool EDGE, class Step, int S>
__device__ __forceinline__ void unit_steps(const AttnParams& p, const Seg& sg, char* ring, Step& st,
                                           int npair, int ulim, int (&q)[S], int& s) {
  using Gm = Geo<KV, D, NW>;
  constexpr int P2 = 2 * Gm::P;
  while (q[0] >= 0 && (EDGE || q[0] <= ulim)) {
    // The unit for the slot this step frees: its page ids are loaded first,
    // while the step's LDS reads are in flight.
    const int un = q[0] + NW * S < npair ? q[0] + NW * S : -1;
    const int an = min(sg.pa + 2 * max(un, 0), sg.pe - 1);
    const int ida = page_id(p, sg.b, an), idb = page_id(p, sg.b, min(an + 1, sg.pe - 1));
    int pending = 0;
#pragma unroll
    for (int i = 1; i < S; ++i) pending += q[i] >= 0;
    wait_steps<P2, S>(pending);
    char* slots = ring + (s % S) * 2 * Gm::SLOT;
    const int a = sg.pa + 2 * q[0];
    st.load(slots, slots + Gm::SLOT);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // LDS reads and page ids
    if (un >= 0) {
      dma_page<KV, D>(p, ida, sg.g, slots);
      dma_page<KV, D>(p, idb, sg.g, slots + Gm::SLOT);
    }
    st.template compute<EDGE>(a, a + 1 < sg.pe);
#pragma unroll
    for (int i = 0; i + 1 < S; ++i) q[i] = q[i + 1];
    q[S - 1] = un;
    ++s;
  }
}

// Streams this wave's pages of the segment through its ring and calls
// st.step(p, slot of page a, slot of page a+1, a, page a+1 exists) for each
// pair of consecutive pages (a = pa + 2u, u = wave, wave + NW, ...).
template <typename KV, int D, int NW, class Step>
__device__ __forceinline__ void run_pages(const AttnParams& p, const Seg& sg, char* ring,
                                          Step& st, bool issued = false) {
  using Gm = Geo<KV, D, NW>;
  constexpr int S = Gm::S, P2 = 2 * Gm::P;
  const int wave = wave_id();
  const int npair = (sg.pe - sg.pa + 1) >> 1;
  if constexpr (Step::kSplit) {
    int q[S];
#pragma unroll
    for (int i = 0; i < S; ++i) q[i] = wave + NW * i < npair ? wave + NW * i : -1;
    if (!issued) issue_first_steps<KV, D, NW>(p, sg, ring, wave, q);
    st.ready();
    // units whose two pages lie inside the committed context (and inside the
    // segment) need no masks
    const int amax = min(sg.S / kPage, sg.pe) - 2;      // last such first page
    const int ulim = amax >= sg.pa ? (amax - sg.pa) >> 1 : -1;
    int s = 0;
    unit_steps<KV, D, NW, false>(p, sg, ring, st, npair, ulim, q, s);
    unit_steps<KV, D, NW, true>(p, sg, ring, st, npair, ulim, q, s);
  } else {
    const int n = npair > wave ? (npair - wave + NW - 1) / NW : 0;
    const int pro = n < S ? n : S;
    for (int s = 0; s < pro; ++s) issue_step<KV, D, NW>(p, sg, ring, wave, s);
    st.ready();
    for (int s = 0; s < n; ++s) {
      wait_steps<P2, S>(min(S - 1, n - 1 - s));
      const char* slots = ring + (s % S) * 2 * Gm::SLOT;
      const int a = sg.pa + 2 * (wave + NW * s);
      st.step(p, slots, slots + Gm::SLOT, a, a + 1 < sg.pe);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this step's LDS reads are done
      if (s + S < n) issue_step<KV, D, NW>(p, sg, ring, wave, s + S);
    }
  }
}

__device__ __forceinline__ uint32_t ld32(const char* a) { return *reinterpret_cast<const uint32_t*>(a); }
__device__ __forceinline__ u32x2 ld64(const char* a) { return *reinterpret_cast<const u32x2*>(a); }
__device__ __forceinline__ u32x4 ld128(const char* a) { return *reinterpret_cast<const u32x4*>(a); }

// Two int8 codes (bytes at bit sh and sh+8 of w) as packed bf16 -- exact: |code| <= 127.
__device__ __forceinline__ uint32_t codes2_to_bf16x2(uint32_t w, int sh) {
  const float a = float(int(w << (24 - sh)) >> 24);
  const float b = float(int(w << (16 - sh)) >> 24);
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}
__device__ __forceinline__ uint32_t ints_to_bf16x2(int lo, int hi) {
  return (__float_as_uint(float(lo)) >> 16) | (__float_as_uint(float(hi)) & 0xffff0000u);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// ============================================================================
// VALU path
// ============================================================================

// Query rows r0 .. r0+15 of the pair into LDS.  fp32 caches: floats
// q[(r*2 + half) * (D/2 + 4) + e]; otherwise bf16 pairs (fp32 Q rounds to
// nearest even) q[(r*2 + half) * (D/4 + 4) + e].  The +4 pads put the two
// halves on different banks.
template <int D, bool F32>
__device__ __forceinline__ void valu_stage_q(const AttnParams& p, const Seg& sg, int r0,
                                             uint32_t* qs) {
  constexpr int HALF = D / 2;
  if constexpr (F32) {
    constexpr int QS = HALF + 4;
    for (int idx = threadIdx.x; idx < kValuRows * D; idx += kWavesValu * kWave) {
      const int r = idx / D, d = idx % D;
      float v = 0.f;
      if (r0 + r < sg.R) {
        const int64_t e = out_row(p, sg, r0 + r) * D + d;
        v = p.q_f32 ? static_cast<const float*>(p.q)[e]
                    : bf16_to_f32(static_cast<const uint16_t*>(p.q)[e]);
      }
      qs[(r * 2 + d / HALF) * QS + d % HALF] = __float_as_uint(v);
    }
  } else {
    constexpr int QS = HALF / 2 + 4;
    for (int idx = threadIdx.x; idx < kValuRows * (D / 2); idx += kWavesValu * kWave) {
      const int r = idx / (D / 2), d2 = idx % (D / 2);       // pair of d = 2*d2, 2*d2+1
      uint32_t w = 0;
      if (r0 + r < sg.R) {
        const int64_t e = out_row(p, sg, r0 + r) * D + 2 * d2;
        if (p.q_f32) {
          const float* qf = static_cast<const float*>(p.q);
          w = pack_bf16x2(qf[e], qf[e + 1]);
        } else {
          w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.q) + e);
        }
      }
      qs[(r * 2 + (2 * d2) / HALF) * QS + d2 % (HALF / 2)] = w;
    }
  }
}

template <typename KV, int D, int RV>
struct ValuStep {
  using Gm = Geo<KV, D, kWavesValu>;      // page geometry only
  static constexpr bool F32 = sizeof(KV) == 4;
  static constexpr bool I8 = sizeof(KV) == 1;
  static constexpr int HALF = D / 2;                  // d values per lane in QK
  static constexpr int QS = F32 ? HALF + 4 : HALF / 2 + 4;
  static constexpr int CPL = D / 64;                  // output columns per lane
  static constexpr bool kSplit = false;               // LDS reads run through the whole step

  const uint32_t* qs;
  char* ps;                                           // [RV][32] probabilities (f32 or bf16)
  float scale_log2;
  float m[RV], l[RV], o[RV][CPL];
  uint32_t vis[RV];                                   // draft masks of the rows
  int ctx;                                            // S of the sequence
  int valid_end;
  int lane, t, h;

  __device__ __forceinline__ ValuStep(const AttnParams& p, const Seg& sg, int r0, const uint32_t* qs_, char* ps_)
      : qs(qs_), ps(ps_) {
    scale_log2 = p.scale_log2;
    lane = lane_id();
    t = lane & 31;
    h = lane >> 5;
    valid_end = sg.S + sg.k;
    ctx = sg.S;
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      m[r] = kNegBig;
      l[r] = 0.f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) o[r][e] = 0.f;
      vis[r] = (r0 + r < sg.R) ? row_mask(p, sg.q0, (r0 + r) / p.G) : 0u;
    }
  }

  // scores of token t for every row: this lane's half of d, both halves summed
  __device__ __forceinline__ void qk(const char* page, int row, float* s) {
    const char* kr = page + row * Gm::RB;
    if constexpr (F32) {
      float kf[HALF];
#pragma unroll
      for (int e = 0; e < Gm::CPR / 2; ++e) {
        const int kappa = h * (Gm::CPR / 2) + e;
        const u32x4 w = ld128(kr + (kappa ^ Gm::swz_k(row)) * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[4 * e + i] = __uint_as_float(w[i]);
      }
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        const uint32_t* q = qs + (r * 2 + h) * QS;
        float a = 0.f;
#pragma unroll
        for (int e4 = 0; e4 < HALF / 4; ++e4) {
          const u32x4 qv = *reinterpret_cast<const u32x4*>(q + 4 * e4);
#pragma unroll
          for (int i = 0; i < 4; ++i) a = fmaf(__uint_as_float(qv[i]), kf[4 * e4 + i], a);
        }
        s[r] = a;
      }
    } else {
      uint32_t kx[HALF / 2];                          // bf16 pairs of this lane's half row
      if constexpr (I8) {
#pragma unroll
        for (int e = 0; e < Gm::CPR / 2; ++e) {       // 16 codes per chunk
          const int kappa = h * (Gm::CPR / 2) + e;
          const u32x4 w = ld128(kr + (kappa ^ Gm::swz_k(row)) * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            kx[8 * e + 2 * i] = codes2_to_bf16x2(w[i], 0);
            kx[8 * e + 2 * i + 1] = codes2_to_bf16x2(w[i], 16);
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < Gm::CPR / 2; ++e) {       // 8 bf16 per chunk
          const int kappa = h * (Gm::CPR / 2) + e;
          const u32x4 w = ld128(kr + (kappa ^ Gm::swz_k(row)) * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) kx[4 * e + i] = w[i];
        }
      }
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        const uint32_t* q = qs + (r * 2 + h) * QS;
        float a = 0.f;
#pragma unroll
        for (int e4 = 0; e4 < HALF / 8; ++e4) {
          const u32x4 qv = *reinterpret_cast<const u32x4*>(q + 4 * e4);
#pragma unroll
          for (int i = 0; i < 4; ++i) a = dot2(kx[4 * e4 + i], qv[i], a);
        }
        s[r] = a;
      }
    }
#pragma unroll
    for (int r = 0; r < RV; ++r) s[r] = xrow32_sum(s[r]);      // the two halves of d
  }

  // O[r][cols] += sum over the 32 tokens of p[r][t] V[t][cols]
  template <bool kMask>
  __device__ __forceinline__ void pv(const char* sa, const char* sb, int a, bool second) {
    if constexpr (F32) {
      const float* pf = reinterpret_cast<const float*>(ps);
#pragma unroll
      for (int t0 = 0; t0 < 32; t0 += 4) {
        float vv[4][CPL];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int tok = t0 + tt, row = tok & 15;
          const char* vr = ((tok < 16) ? sa : sb) + Gm::PAGE + row * Gm::RB;
          const int cb = lane * CPL * 4;
          const char* src = vr + ((cb / 16) ^ Gm::swz_v(row)) * 16 + cb % 16;
#pragma unroll
          for (int e = 0; e < CPL; ++e) vv[tt][e] = reinterpret_cast<const float*>(src)[e];
          if constexpr (kMask) {
            const bool ok = (tok < 16 || second) && ((a + (tok >> 4)) * kPage + row < valid_end);
#pragma unroll
            for (int e = 0; e < CPL; ++e) vv[tt][e] = ok ? vv[tt][e] : 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < RV; ++r) {
          const f32x4 pw = *reinterpret_cast<const f32x4*>(pf + r * 32 + t0);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int e = 0; e < CPL; ++e) o[r][e] = fmaf(pw[tt], vv[tt][e], o[r][e]);
          }
        }
      }
    } else {
#pragma unroll
      for (int tq = 0; tq < 16; tq += 4) {            // 4 token pairs = 8 tokens
        uint32_t vp[4][CPL];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int tok = 2 * (tq + u), row = tok & 15;
          const char* vr = ((tok < 16) ? sa : sb) + Gm::PAGE;
          const char* r0p = vr + row * Gm::RB;
          const char* r1p = vr + (row + 1) * Gm::RB;
          if constexpr (I8) {
            const int cb = lane * CPL;                // byte of this lane's first column
            const int kap = cb / 16, wi = cb % 16;
            const char* s0 = r0p + (kap ^ Gm::swz_v(row)) * 16 + wi;
            const char* s1 = r1p + (kap ^ Gm::swz_v(row + 1)) * 16 + wi;
            if constexpr (CPL == 2) {
              const int c00 = reinterpret_cast<const int8_t*>(s0)[0];
              const int c01 = reinterpret_cast<const int8_t*>(s0)[1];
              const int c10 = reinterpret_cast<const int8_t*>(s1)[0];
              const int c11 = reinterpret_cast<const int8_t*>(s1)[1];
              vp[u][0] = ints_to_bf16x2(c00, c10);
              vp[u][CPL - 1] = ints_to_bf16x2(c01, c11);
            } else {
              vp[u][0] = ints_to_bf16x2(reinterpret_cast<const int8_t*>(s0)[0],
                                        reinterpret_cast<const int8_t*>(s1)[0]);
            }
          } else {
            const int cb = lane * CPL * 2;
            const int kap = cb / 16, wi = cb % 16;
            const char* s0 = r0p + (kap ^ Gm::swz_v(row)) * 16 + wi;
            const char* s1 = r1p + (kap ^ Gm::swz_v(row + 1)) * 16 + wi;
            if constexpr (CPL == 2) {
              const uint32_t w0 = ld32(s0), w1 = ld32(s1);
              vp[u][0] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
              vp[u][CPL - 1] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
            } else {
              vp[u][0] = uint32_t(*reinterpret_cast<const uint16_t*>(s0)) |
                         (uint32_t(*reinterpret_cast<const uint16_t*>(s1)) << 16);
            }
            if constexpr (kMask) {
              const int pos0 = (a + (tok >> 4)) * kPage + row;
              const bool pg_ok = tok < 16 || second;
              const uint32_t keep = ((pg_ok && pos0 < valid_end) ? 0x0000ffffu : 0u) |
                                    ((pg_ok && pos0 + 1 < valid_end) ? 0xffff0000u : 0u);
#pragma unroll
              for (int e = 0; e < CPL; ++e) vp[u][e] &= keep;
            }
          }
        }
#pragma unroll
        for (int r = 0; r < RV; ++r) {
          const u32x4 pp = ld128(ps + r * 64 + tq * 4);  // probability pairs of 4 token pairs
#pragma unroll
          for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int e = 0; e < CPL; ++e) o[r][e] = dot2(pp[u], vp[u][e], o[r][e]);
          }
        }
      }
    }
  }

  __device__ __forceinline__ void step(const AttnParams&, const char* sa, const char* sb, int a,
                                       bool second) {
    const char* page = (t < 16) ? sa : sb;
    const int row = t & 15;
    const int pos = (a + (t >> 4)) * kPage + row;
    const bool tok_ok = (t < 16) || second;
    float s[RV];
    qk(page, row, s);
    float ksc = 1.f, vsc = 1.f;
    if constexpr (I8) {
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(page + 2 * Gm::PAGE);
      ksc = f16_bits_to_f32(sc[row]);
      vsc = (tok_ok && pos < valid_end) ? f16_bits_to_f32(sc[16 + row]) : 0.f;
    }
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const float x = (tok_ok && key_visible(pos, ctx, valid_end, vis[r])) ? s[r] * scale_log2 * ksc : -INFINITY;
      const float mx = xrow16_max(row16_max(x));                // over the 32 tokens
      const float mn = fmaxf(m[r], mx);
      const float alpha = exp2f(m[r] - mn);
      m[r] = mn;
      const float e = exp2f(x - mn);
      l[r] = l[r] * alpha + e;
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[r][c] *= alpha;
      if (h == 0) {
        if constexpr (F32) reinterpret_cast<float*>(ps)[r * 32 + t] = e * vsc;
        else reinterpret_cast<uint16_t*>(ps)[r * 32 + t] = f32_to_bf16(e * vsc);
      }
    }
    wave_sync();
    // garbage rows exist only in the pair's last page and in a missing second page
    const bool mask = !second || (a + 2) * kPage > valid_end;
    if (mask) pv<true>(sa, sb, a, second);
    else pv<false>(sa, sb, a, second);
    wave_sync();
  }

  // Queries come from LDS, nothing to wait for.
  __device__ __forceinline__ void ready() const {}
  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int r = 0; r < RV; ++r) l[r] = xrow16_sum(row16_sum(l[r]));
  }

  static constexpr int SLOT_F = RV * kWave * CPL + 2 * RV;
  __device__ __forceinline__ void store(float* slot) const {
#pragma unroll
    for (int r = 0; r < RV; ++r) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) slot[(r * kWave + lane) * CPL + e] = o[r][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        slot[RV * kWave * CPL + r] = m[r];
        slot[RV * kWave * CPL + RV + r] = l[r];
      }
    }
  }
  __device__ __forceinline__ void combine(const float* slot) {
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const float mo = slot[RV * kWave * CPL + r];
      const float lo = slot[RV * kWave * CPL + RV + r];
      const float M = fmaxf(m[r], mo);
      const float fa = exp2f(m[r] - M), fb = exp2f(mo - M);
      l[r] = fa * l[r] + fb * lo;
      m[r] = M;
#pragma unroll
      for (int e = 0; e < CPL; ++e) o[r][e] = fa * o[r][e] + fb * slot[(r * kWave + lane) * CPL + e];
    }
  }
  __device__ __forceinline__ void write(const AttnParams& p, const Seg& sg, int r0) const {
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const int rr = r0 + r;
      if (rr >= sg.R) continue;
      if (sg.full) {
        const float inv = 1.f / l[r];
        const int64_t oe = out_row(p, sg, rr) * D + lane * CPL;
#pragma unroll
        for (int e = 0; e < CPL; ++e) store_out1(p, oe + e, o[r][e] * inv);
      } else {
        float* sb = slot_base<D>(p, sg.slot);
#pragma unroll
        for (int e = 0; e < CPL; ++e) st_dev(sb + int64_t(rr) * D + lane * CPL + e, o[r][e]);
        if (lane == 0) {
          st_dev(sb + int64_t(p.slot_rows) * D + rr, m[r]);
          st_dev(sb + int64_t(p.slot_rows) * (D + 1) + rr, l[r]);
        }
      }
    }
  }
};

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

// 8 bf16 values (as packed words) times `mul` -> fp16, one rounding to nearest
// even from the fp32 product.
__device__ __forceinline__ f16x8 bf16x8_to_f16(u32x4 w, float mul) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack_f16x2(__uint_as_float(w[i] << 16) * mul, __uint_as_float(w[i] & 0xffff0000u) * mul);
  return __builtin_bit_cast(f16x8, r);
}

// 8 consecutive Q values times `mul` as fp16 (the INT8 path's operand type;
// one rounding to nearest even from the fp32 product).
__device__ __forceinline__ f16x8 load_q8_f16(const AttnParams& p, int64_t elem, float mul) {
  float v[8];
  if (p.q_f32) {
    const f32x4* s = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) + elem);
    const f32x4 a = s[0], b = s[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_f16x2(v[2 * i] * mul, v[2 * i + 1] * mul);
  return __builtin_bit_cast(f16x8, r);
}

// 8 INT8 codes -> fp16 values 1152 + code, exactly: code ^ 0x80 is code + 128
// as an unsigned byte u, and the fp16 bit pattern 0x6400 | u is 1024 + u.
__device__ __forceinline__ f16x8 codes8_to_f16(uint32_t w0, uint32_t w1) {
  const uint32_t a = w0 ^ 0x80808080u, b = w1 ^ 0x80808080u;
  const uint32_t k = 0x64646464u;
  const u32x4 r = {__builtin_amdgcn_perm(k, a, 0x04010400u), __builtin_amdgcn_perm(k, a, 0x04030402u),
                   __builtin_amdgcn_perm(k, b, 0x04010400u), __builtin_amdgcn_perm(k, b, 0x04030402u)};
  return __builtin_bit_cast(f16x8, r);
}

// One step of the MFMA path over two pages (32 tokens) for up to 16*NRB query
// rows.  Lane (l16, c) = (lane % 16, lane / 16).
//  * S^T = K Q^T, v_mfma_f32_16x16x32: the lane holds tokens 4c..4c+3 of each
//    page for query row l16.
//  * Online softmax with a lazy reference maximum: a row's reference moves
//    (and its accumulators are rescaled) only when a score exceeds it by more
//    than kLazy in log2 units, so weights stay below 2^kLazy and rescaling is
//    rare; results are those of the exact maximum up to rounding.
//  * O^T += V^T P^T, v_mfma_f32_16x16x32 over both pages: k-slot e of lane
//    group c is token 4c + e%4 of page e/4 on both operands.  V^T comes
//    straight from LDS with the transposing reads ds_read_b64_tr_b16 (bf16) and
//    ds_read_b64_tr_b8 (INT8).
//  * The softmax denominator of the bf16 path comes from the same MFMA with an
//    all-ones A operand, so it sums exactly the rounded weights P.V uses.
//  * INT8 caches run fp16 MFMAs on codes offset to 1152 + code (exact); the
//    offset leaves S through the accumulator's start value -1152 * sum(q) and
//    leaves O through the MFMA-computed sum of the fp16 weights.  Q is
//    converted once, pre-multiplied by softmax_scale * log2 e, so the per-token
//    K scale is the only factor left on each score; the V scale multiplies the
//    fp16 weight pairs, and the denominator is a second all-ones MFMA over the
//    unscaled weights.
template <typename KV, int D, int NRB, bool kIdx = false>
struct MfmaStep {
  using Gm = Geo<KV, D, kWavesValu>;      // page geometry only
  static constexpr bool I8 = sizeof(KV) == 1;
  using Op8 = typename std::conditional<I8, f16x8, bf16x8>::type;
  static constexpr int KS = D / 32;       // 16x16x32 k-steps over d (S^T)
  static constexpr int NDB = D / 16;      // 16-column blocks of d (O^T)
  static constexpr float kLazy = 8.f;
  static constexpr float kCodeBias = 1152.f;
  static constexpr bool kSplit = true;
  // V^T operand as read from LDS: bf16 -- the operand itself; INT8 -- 8 codes
  using VRaw = typename std::conditional<I8, i32x2, bf16x8>::type;

  Op8 qB[NRB][KS];                        // row 16 rb + l16, d 32c + 8ks .. +8
  f32x4 acc[NRB][NDB];                    // O^T: d 16 db + 4c + i, row 16 rb + l16
  f32x4 sacc[NRB];                        // all-ones MFMA: sum of the weights fed to P.V
  f32x4 lsum[NRB];                        // INT8: all-ones MFMA over the unscaled weights
  float m[NRB], l[NRB];
  float s0[NRB];                          // INT8: start value of the S^T accumulator
  // draft visibility of the rows: masks, or draft indices (kIdx)
  typename std::conditional<kIdx, int, uint32_t>::type vis[NRB];
  int ctx;                                // S of the sequence
  int valid_end;
  int lane, l16, c;
  bool qbf16;                             // INT8 with bf16 Q: qB holds bf16 until ready()
  float scale_log2;
  // carried from load() to compute()
  f32x4 s[2][NRB];                        // S^T of both pages (unscaled)
  VRaw vr[NDB];                           // V^T operands (INT8: codes)
  u32x2 kw[2], vw[2];                     // INT8: K and V scales of lane's 4 tokens

  static __device__ __forceinline__ f32x4 mfma32(Op8 a, Op8 b, f32x4 acc) {
    if constexpr (I8) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
  static __device__ __forceinline__ Op8 ones() {
    const uint32_t one = I8 ? 0x3c003c00u : 0x3f803f80u;
    return __builtin_bit_cast(Op8, u32x4{one, one, one, one});
  }

  __device__ __forceinline__ MfmaStep(const AttnParams& p, const Seg& sg, int r0) {
    scale_log2 = p.scale_log2;
    lane = lane_id();
    l16 = lane & 15;
    c = lane >> 4;
    valid_end = sg.S + sg.k;
    ctx = sg.S;
    // bf16 Q is only loaded here (raw words); work that needs the values waits
    // for ready(), after the first page copies are issued.
    qbf16 = I8 && !p.q_f32;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = r0 + 16 * rb + l16;
      vis[rb] = kIdx ? -1 : 0;
      if (r < sg.R) {
        if constexpr (kIdx) vis[rb] = r / p.G;
        else vis[rb] = row_mask(p, sg.q0, r / p.G);
        const int64_t qe = out_row(p, sg, r) * D + c * (D / 4);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (p.q_f32) {
            if constexpr (I8) qB[rb][ks] = load_q8_f16(p, qe + 8 * ks, scale_log2);
            else qB[rb][ks] = load_q8_bf16(p, qe + 8 * ks);
          } else {
            qB[rb][ks] = __builtin_bit_cast(
                Op8, *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) + qe + 8 * ks));
          }
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qB[rb][ks] = __builtin_bit_cast(Op8, u32x4{0, 0, 0, 0});
      }
      m[rb] = kNegBig;
      l[rb] = 0.f;
      sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      lsum[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  __device__ __forceinline__ bool visible(int pos, int rb) const {
    if constexpr (kIdx) return key_visible_idx(pos, ctx, valid_end, vis[rb]);
    else return key_visible(pos, ctx, valid_end, vis[rb]);
  }

  // A operand of S^T = K Q^T: K row l16, d 32c + 8ks .. +8
  __device__ __forceinline__ Op8 k_operand(const char* page, int ks) const {
    const char* kr = page + l16 * Gm::RB;
    if constexpr (I8) {
      const int byte = c * (D / 4) + 8 * ks;
      const u32x2 w = ld64(kr + ((byte / 16) ^ Gm::swz_k(l16)) * 16 + byte % 16);
      return codes8_to_f16(w[0], w[1]);
    } else {
      const int kappa = c * (Gm::CPR / 4) + ks;
      return __builtin_bit_cast(bf16x8, ld128(kr + (kappa ^ Gm::swz_k(l16)) * 16));
    }
  }

  // A operand of O^T += V^T P^T for d columns 16db .. 16db+15: lane (l16, c)
  // receives V[token 4c + e%4 of page e/4][16 db + l16], e = 0..7.
  __device__ __forceinline__ VRaw v_raw(const char* sa, const char* sb, int db) const {
    if constexpr (I8) {
      // ds_read_b64_tr_b8: lane j of a 16-lane group receives byte e from the
      // 8-byte block addressed by lane 2e + j/8, at column j%8.  Lane 2e + h
      // therefore addresses V[token e][16 db + 8h .. +8].
      const int e = l16 >> 1, h = l16 & 1;
      const int rho = 4 * c + (e & 3);
      const char* src = (e < 4 ? sa : sb) + Gm::PAGE + rho * Gm::RB +
                        (db ^ Gm::swz_v(rho)) * 16 + 8 * h;
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32((AS3 i32x2*)src);
    } else {
      // ds_read_b64_tr_b16: lane j of a 16-lane group receives element e from
      // the 8-byte block addressed by lane 4e + j/4, at column j%4.  Lane 4e + q
      // therefore addresses V[row 4c + e][16 db + 4q .. +4], once per page.
      const int e = l16 >> 2, q = l16 & 3;
      const int rho = 4 * c + e;
      const int off = Gm::PAGE + rho * Gm::RB + ((2 * db + (q >> 1)) ^ Gm::swz_v(rho)) * 16 +
                      8 * (q & 1);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((AS3 bf16x4*)(sa + off));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((AS3 bf16x4*)(sb + off));
      const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
      return __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
    }
  }
  static __device__ __forceinline__ Op8 v_operand(VRaw r) {
    if constexpr (I8) return codes8_to_f16(uint32_t(r[0]), uint32_t(r[1]));
    else return r;
  }

  // Every LDS read of a step: K operands (fed straight into the S^T MFMAs),
  // the V^T operands and the INT8 scales.  Both slots are always multiplied:
  // without a second page, slot B holds a copy of page A (finite data) whose
  // scores are masked to -inf later.  A branch around these products would put
  // a read of their accumulators right after a taken jump, where this compiler
  // omits the MFMA result wait states.
  // S^T of the pages in slots sa, sb (one unit) into dst.
  __device__ __forceinline__ void scores(const char* sa, const char* sb,
                                         f32x4 (&dst)[2][NRB]) const {
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float z = I8 ? s0[rb] : 0.f;
        dst[pg][rb] = f32x4{z, z, z, z};
      }
      const char* page = pg ? sb : sa;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const Op8 ka = k_operand(page, ks);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) dst[pg][rb] = mfma32(ka, qB[rb][ks], dst[pg][rb]);
      }
    }
  }

  __device__ __forceinline__ void load(const char* sa, const char* sb) {
    scores(sa, sb, s);
#pragma unroll
    for (int db = 0; db < NDB; ++db) vr[db] = v_raw(sa, sb, db);
    if constexpr (I8) {
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        const char* sc = (pg ? sb : sa) + 2 * Gm::PAGE;
        kw[pg] = ld64(sc + 8 * c);
        vw[pg] = ld64(sc + 32 + 8 * c);
      }
    }
  }

  // Softmax and P.V of the step over pages a, a+1.  EDGE = false: all 32
  // tokens lie inside the committed context, so every query row sees them and
  // none is a garbage row -- no masks.
  template <bool EDGE>
  __device__ __forceinline__ void compute(int a, bool second) {
    // The values the rest depends on pass through an empty asm here, so none
    // of this work is hoisted above the copy issued just before it.
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) asm volatile("" : "+v"(s[pg][rb]));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(vr[db]));
    if constexpr (I8) {
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) asm volatile("" : "+v"(kw[pg]), "+v"(vw[pg]));
    }
    if constexpr (I8) softmax_pv_i8<EDGE>(a, second);
    else softmax_pv<EDGE>(a, second, s);
  }

  // INT8 caches.  Q carries softmax_scale * log2 e, so a token's score in log2
  // units is s * k_scale, and y = s * k_scale - m is one v_fma_mix_f32 with the
  // fp16 scale as an operand.  Weights: e = 2^y packed to fp16 (the unscaled
  // weights, whose all-ones MFMA gives the denominator), then times the fp16
  // V scale pair (the P operand, whose all-ones MFMA gives the sum that
  // removes the code offset).
  template <bool EDGE>
  __device__ __forceinline__ void softmax_pv_i8(int a, bool second) {
    const int npg = second ? 2 : 1;
    Op8 va[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) va[db] = v_operand(vr[db]);
    // V scales of the lane's tokens as fp16 pairs, in k-slot order
    uint32_t vs[4] = {vw[0][0], vw[0][1], vw[1][0], vw[1][1]};
    if constexpr (EDGE) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {        // garbage rows (scale may be NaN) weigh zero
        const int p0 = (a + (h >> 1)) * kPage + 4 * c + 2 * (h & 1);
        vs[h] &= (p0 < valid_end ? 0x0000ffffu : 0u) | (p0 + 1 < valid_end ? 0xffff0000u : 0u);
      }
    }
    float y[NRB][8];
    bool move = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float t = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int pg = j >> 2, i = j & 3;
        const int pos = (a + pg) * kPage + 4 * c + i;
        const float v = fmaf(s[pg][rb][i], f16x2_half(kw[pg][i >> 1], i & 1), -m[rb]);
        y[rb][j] = (!EDGE || (pg < npg && visible(pos, rb))) ? v : -INFINITY;
        t = fmaxf(t, y[rb][j]);
      }
      move |= xrow32_max(xrow16_max(t)) > kLazy;
    }
    if (__ballot(move)) {          // some row's reference moves: exact maxima of this step
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float x[8], t = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int pg = j >> 2, i = j & 3;
          const int pos = (a + pg) * kPage + 4 * c + i;
          const float v = s[pg][rb][i] * f16x2_half(kw[pg][i >> 1], i & 1);
          x[j] = (!EDGE || (pg < npg && visible(pos, rb))) ? v : -INFINITY;
          t = fmaxf(t, x[j]);
        }
        const float xm = xrow32_max(xrow16_max(t));
        const float mn = (xm > m[rb] + kLazy) ? xm : m[rb];
        const float alpha = __builtin_amdgcn_exp2f(m[rb] - mn);
        m[rb] = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sacc[rb][i] *= alpha;
          lsum[rb][i] *= alpha;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][db][i] *= alpha;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) y[rb][j] = x[j] - mn;
      }
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      u32x4 pe, pw;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        pe[h] = pack_f16x2(__builtin_amdgcn_exp2f(y[rb][2 * h]), __builtin_amdgcn_exp2f(y[rb][2 * h + 1]));
        pw[h] = mul_f16x2(pe[h], vs[h]);
      }
      const Op8 pb = __builtin_bit_cast(Op8, pw);
      lsum[rb] = mfma32(ones(), __builtin_bit_cast(Op8, pe), lsum[rb]);
      sacc[rb] = mfma32(ones(), pb, sacc[rb]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[rb][db] = mfma32(va[db], pb, acc[rb][db]);
    }
  }

  // bf16 caches: scores times scale * log2 e, lazy maximum, bf16 weights.
  template <bool EDGE>
  __device__ __forceinline__ void softmax_pv(int a, bool second, const f32x4 (&sc)[2][NRB]) {
    const int npg = second ? 2 : 1;
    Op8 va[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) va[db] = v_operand(vr[db]);
    if constexpr (EDGE) {
      if ((a + 2) * kPage > valid_end) {          // garbage rows (may be NaN) read as zero
        u32x4 keep;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int p0 = (a + (h >> 1)) * kPage + 4 * c + 2 * (h & 1);
          keep[h] = (p0 < valid_end ? 0x0000ffffu : 0u) | (p0 + 1 < valid_end ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          va[db] = __builtin_bit_cast(Op8, __builtin_bit_cast(u32x4, va[db]) & keep);
      }
    }
    // Masked scores and row maxima of every row block first, then one
    // wave-uniform decision for all of them, so that the blocks' work stays
    // straight-line code the compiler can interleave.  The maxima are taken
    // over the unscaled scores (scale_log2 > 0: see ready()) and scaled once
    // per row; each weight is then exp2 of one fma.
    float x[NRB][2][4], mx[NRB];
    bool move = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float t = -INFINITY;
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = (a + pg) * kPage + 4 * c + i;
          x[rb][pg][i] = (!EDGE || (pg < npg && visible(pos, rb))) ? sc[pg][rb][i] : -INFINITY;
          t = fmaxf(t, x[rb][pg][i]);
        }
      }
      mx[rb] = xrow32_max(xrow16_max(t)) * scale_log2;          // over the 4 lanes of the row
      move |= mx[rb] > m[rb] + kLazy;
    }
    if (__ballot(move)) {                                       // some row's reference moves
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float mn = (mx[rb] > m[rb] + kLazy) ? mx[rb] : m[rb];
        const float alpha = __builtin_amdgcn_exp2f(m[rb] - mn);
        m[rb] = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[rb][i] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][db][i] *= alpha;
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      u32x4 pw;
#pragma unroll
      for (int h = 0; h < 4; ++h)
        pw[h] = pack_bf16x2(
            __builtin_amdgcn_exp2f(fmaf(x[rb][h >> 1][2 * (h & 1)], scale_log2, -m[rb])),
            __builtin_amdgcn_exp2f(fmaf(x[rb][h >> 1][2 * (h & 1) + 1], scale_log2, -m[rb])));
      const Op8 pb = __builtin_bit_cast(Op8, pw);
      sacc[rb] = mfma32(ones(), pb, sacc[rb]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[rb][db] = mfma32(va[db], pb, acc[rb][db]);
    }
  }

  // Called once the first pages are in flight: the query registers are read
  // here, so the compiler's wait for their loads lands outside the page loop
  // (one wait that also covers the first DMAs) instead of inside it.
  // INT8: fp16 operands from bf16 Q (times softmax_scale * log2 e), and the S^T
  // start value -1152 * sum(q).
  // bf16: a negative softmax scale is moved into Q (a sign flip, exact), so
  // the score maxima can be taken before scaling.
  __device__ __forceinline__ void ready() {
    const bool flip = !I8 && scale_log2 < 0.f;
    if (flip) scale_log2 = -scale_log2;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if constexpr (!I8) {
        if (flip) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            qB[rb][ks] = __builtin_bit_cast(
                Op8, __builtin_bit_cast(u32x4, qB[rb][ks]) ^ u32x4{0x80008000u, 0x80008000u,
                                                                   0x80008000u, 0x80008000u});
        }
      }
      if constexpr (I8) {
        if (qbf16) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            qB[rb][ks] = bf16x8_to_f16(__builtin_bit_cast(u32x4, qB[rb][ks]), scale_log2);
        }
        float qs = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 w = __builtin_bit_cast(u32x4, qB[rb][ks]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            qs += f16_bits_to_f32(uint16_t(w[i])) + f16_bits_to_f32(uint16_t(w[i] >> 16));
        }
        s0[rb] = -kCodeBias * xrow32_sum(xrow16_sum(qs));
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qB[rb][ks]));
    }
  }
  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if constexpr (I8) {
        l[rb] = lsum[rb][0];
        const float off = kCodeBias * sacc[rb][0];             // remove 1152 * sum of weights
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][db][i] -= off;
        }
      } else {
        l[rb] = sacc[rb][0];
      }
    }
  }

  static constexpr int SLOT_F = NRB * NDB * kWave * 4 + 2 * NRB * kWave;
  static constexpr int SLOT_ROWS = 16 * NRB;
  __device__ __forceinline__ void store(float* slot) const {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(slot + ((rb * NDB + db) * kWave + lane) * 4) = acc[rb][db];
      slot[NRB * NDB * kWave * 4 + rb * kWave + lane] = m[rb];
      slot[NRB * NDB * kWave * 4 + (NRB + rb) * kWave + lane] = l[rb];
    }
  }
  // Normalised output rows r0 .. r0 + 16 NRB - 1 (those below sg.R) straight
  // from this wave's state (row-block kernel: every wave owns its rows).
  __device__ __forceinline__ void write_rows(const AttnParams& p, const Seg& sg, int r0) const {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = r0 + 16 * rb + l16;
      if (r >= sg.R) continue;
      const float inv = 1.f / l[rb];
      const int64_t oe = out_row(p, sg, r) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x4 v = acc[rb][db];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= inv;
        store_out4(p, oe + 16 * db + 4 * c, v);
      }
    }
  }

  // This wave's partial state -- unnormalised O, running maxima, weight sums
  // -- of rows rr0 .. rr0 + 16 NRB - 1 of a slot of slot_rows rows laid out
  // as O [slot_rows][D], m [slot_rows], l [slot_rows] (row-block key slices).
  __device__ __forceinline__ void write_partial(float* slot, int rr0, int slot_rows) const {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int rr = rr0 + 16 * rb + l16;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(slot + rr * D + 16 * db + 4 * c) = acc[rb][db];
      if (c == 0) {
        slot[slot_rows * D + rr] = m[rb];
        slot[slot_rows * (D + 1) + rr] = l[rb];
      }
    }
  }

  // One (row, 4-column) item of the merge of the nw waves' states stored at
  // mrg + w * stride (store() layout), combined in wave order: the running
  // maximum M, the denominator L and the unnormalised output columns O.
  static __device__ __forceinline__ void merge_item(const float* mrg, int nw, int stride, int r,
                                                    int d4, float& M, float& L, f32x4& O) {
    constexpr int MOFF = NRB * NDB * kWave * 4;
    const int oidx = (((r >> 4) * NDB + (d4 >> 2)) * kWave + (r & 15) + 16 * (d4 & 3)) * 4;
    const int midx = MOFF + (r >> 4) * kWave + (r & 15);
    M = kNegBig;
    for (int w = 0; w < nw; ++w) M = fmaxf(M, mrg[w * stride + midx]);
    L = 0.f;
    O = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < nw; ++w) {
      const float* sl = mrg + w * stride;
      const float f = exp2f(sl[midx] - M);
      L += f * sl[midx + NRB * kWave];
      const f32x4 o = *reinterpret_cast<const f32x4*>(sl + oidx);
#pragma unroll
      for (int i = 0; i < 4; ++i) O[i] += f * o[i];
    }
  }
  // The same merge in two phases, for the 8-wave INT8 kernel, where reading
  // every wave's (m, l) once per item makes the merge LDS-bound.  Rows: threads 0 .. 16 NRB - 1 each take one query row and
  // write to tab (kMergeTab floats per row) the wave weights f_w = 2^(m_w - M)
  // in entries 0 .. nw-1, the running maximum M (entry 8) and the denominator
  // L = sum_w f_w l_w (entry 9), in wave order.  Columns (after a barrier):
  // each (row, 4-column) item sums f_w O_w in wave order.
  static __device__ __forceinline__ void merge_rows(const float* mrg, int nw, int stride,
                                                    float* tab, int tid) {
    constexpr int MOFF = NRB * NDB * kWave * 4;
    if (tid >= 16 * NRB) return;
    const int midx = MOFF + (tid >> 4) * kWave + (tid & 15);
    float M = kNegBig;
    for (int w = 0; w < nw; ++w) M = fmaxf(M, mrg[w * stride + midx]);
    float L = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float f = exp2f(mrg[w * stride + midx] - M);
      L += f * mrg[w * stride + midx + NRB * kWave];
      tab[tid * kMergeTab + w] = f;
    }
    tab[tid * kMergeTab + 8] = M;
    tab[tid * kMergeTab + 9] = L;
  }
  static __device__ __forceinline__ void merge_cols(const float* mrg, int nw, int stride,
                                                    const float* tab, int r, int d4, float& M,
                                                    float& L, f32x4& O) {
    const int oidx = (((r >> 4) * NDB + (d4 >> 2)) * kWave + (r & 15) + 16 * (d4 & 3)) * 4;
    O = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < nw; ++w) {
      const float f = tab[r * kMergeTab + w];
      const f32x4 o = *reinterpret_cast<const f32x4*>(mrg + w * stride + oidx);
#pragma unroll
      for (int i = 0; i < 4; ++i) O[i] += f * o[i];
    }
    M = tab[r * kMergeTab + 8];
    L = tab[r * kMergeTab + 9];
  }
  // Unnormalised partial (O, m, l) of row `row` of a segment that is not the
  // whole pair, into the segment's slot (device-coherent stores).
  static __device__ __forceinline__ void write_partial(const AttnParams& p, const Seg& sg, int row,
                                                       int d4, float M, float L, const f32x4& O) {
    float* sb = slot_base<D>(p, sg.slot);
    st_dev4(slot_rsrc(sb, p.slot_rows * D * 4), (row * D + 4 * d4) * 4, O);
    if (d4 == 0) {
      st_dev(sb + int64_t(p.slot_rows) * D + row, M);
      st_dev(sb + int64_t(p.slot_rows) * (D + 1) + row, L);
    }
  }

  // Every item of the wave merge (two phases in the INT8 kernel: the
  // barrier between them is called by every thread).
  static __device__ __forceinline__ void merge_any(const float* mrg, int nw, int stride, int r,
                                                   int d4, float& M, float& L, f32x4& O) {
    if constexpr (I8) merge_cols(mrg, nw, stride, merge_table(), r, d4, M, L, O);
    else merge_item(mrg, nw, stride, r, d4, M, L, O);
  }
  static __device__ __forceinline__ void merge_prepare(const float* mrg, int nw, int stride,
                                                       int tid) {
    if constexpr (I8) {
      merge_rows(mrg, nw, stride, merge_table(), tid);
      __syncthreads();
    }
  }

  // Merge of the nw waves' states spread over every thread of the workgroup:
  // thread items are (row, 4 columns), rows varying fastest so that a wave's
  // 16-byte LDS reads spread over all banks; writes the normalised output
  // rows, or the partial of a segment that is not the whole pair.
  static __device__ __forceinline__ void merge_write(const AttnParams& p, const Seg& sg, int r0,
                                                     const float* mrg, int nw, int stride) {
    constexpr int ITEMS = 16 * NRB * (D / 4);
    merge_prepare(mrg, nw, stride, merge_tid<I8>());
    for (int it = merge_tid<I8>(); it < ITEMS; it += nw * kWave) {
      const int r = it % (16 * NRB), d4 = it / (16 * NRB);
      float M, L;
      f32x4 O;
      merge_any(mrg, nw, stride, r, d4, M, L, O);
      const int row = r0 + r;
      if (row >= sg.R) continue;                    // padding rows of the last block
      if (sg.full) {
        const float inv = 1.f / L;
#pragma unroll
        for (int i = 0; i < 4; ++i) O[i] *= inv;
        store_out4(p, out_row(p, sg, row) * D + 4 * d4, O);
      } else {
        write_partial(p, sg, row, d4, M, L, O);
      }
    }
  }
};


// ---- phase-split form of the MFMA step (row-block kernel) -----------------
// The arithmetic of MfmaStep (NRB = 2: 32 query rows per wave) on groups of
// NU units (2 NU pages), cut where the products of a group end and its
// softmax begins: mma_phase() runs every matrix product of a phase -- P.V of
// the previous group from the weights held in pw / pe, then S^T of the
// current group -- and softmax_phase() turns S^T into those weights (one
// reference update per group).  Two waves sharing a SIMD can then run one's
// products beside the other's softmax.
template <typename KV, int D, int NU, bool kIdx>
struct PhaseStep : MfmaStep<KV, D, 2, kIdx> {
  using Base = MfmaStep<KV, D, 2, kIdx>;
  using Op8 = typename Base::Op8;
  using Gm = typename Base::Gm;
  static constexpr bool I8 = Base::I8;
  static constexpr int NRB = 2;
  static constexpr int NDB = Base::NDB;
  static constexpr int NP = 2 * NU;       // pages per group
  static constexpr float kLazy = Base::kLazy;
  using Base::acc;
  using Base::sacc;
  using Base::lsum;
  using Base::m;
  using Base::c;
  using Base::valid_end;
  using Base::scale_log2;

  f32x4 sp[NP][NRB];                      // S^T of the group (unscaled)
  u32x4 pw[NU][NRB];                      // P operands of the last softmax phase
  u32x4 pe[NU][NRB];                      // INT8: the unscaled weights (denominator)
  u32x2 kwp[NP], vwp[NP];                 // INT8: K and V scales of lane's 4 tokens

  __device__ __forceinline__ PhaseStep(const AttnParams& p, const Seg& sg, int r0)
      : Base(p, sg, r0) {}

  // pages of a group: NP consecutive ring slots from `base`
  static __device__ __forceinline__ const char* page(const char* base, int j) {
    return base + j * Gm::SLOT;
  }

  // Steady groups (kSteady: both groups exist, no masks) order the phase's
  // instructions explicitly: a wave keeps at most 15 LDS reads in flight and
  // each takes about 300 clocks to return (measured on gfx950 with the
  // operand patterns here), so the reads go out a few ahead and then one
  // between consecutive MFMAs, instead of in one block the wave then waits
  // on (the 7B-shaped long step: about 4 % faster in A/B runs).
  static constexpr int kPhaseReads = NU * NDB * 2 + NP * Base::KS;          // V, K
  static constexpr int kPhaseMfma = NU * NRB * (NDB + 1) + NP * Base::KS * NRB;
  static constexpr int kReadsAhead = 8;

  template <bool EDGE, bool kSteady = false>
  __device__ __forceinline__ void mma_phase(const char* prev_base, int a_prev, bool prev,
                                            const char* cur_base, bool cur) {
    if (kSteady || prev) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const char* sa = page(prev_base, 2 * u);
        const char* sb = page(prev_base, 2 * u + 1);
        Op8 va[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) va[db] = Base::v_operand(this->v_raw(sa, sb, db));
        if constexpr (EDGE && !I8) {
          const int a = a_prev + 2 * u;
          if ((a + 2) * kPage > valid_end) {        // garbage rows (may be NaN) read as zero
            u32x4 keep;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const int p0 = (a + (h >> 1)) * kPage + 4 * c + 2 * (h & 1);
              keep[h] = (p0 < valid_end ? 0x0000ffffu : 0u) | (p0 + 1 < valid_end ? 0xffff0000u : 0u);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              va[db] = __builtin_bit_cast(Op8, __builtin_bit_cast(u32x4, va[db]) & keep);
          }
        }
        // each V operand feeds its row blocks back to back
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            acc[rb][db] = Base::mfma32(va[db], __builtin_bit_cast(Op8, pw[u][rb]), acc[rb][db]);
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          if constexpr (I8)
            lsum[rb] = Base::mfma32(Base::ones(), __builtin_bit_cast(Op8, pe[u][rb]), lsum[rb]);
          sacc[rb] = Base::mfma32(Base::ones(), __builtin_bit_cast(Op8, pw[u][rb]), sacc[rb]);
        }
      }
    }
    if (kSteady || cur) {
#pragma unroll
      for (int pg = 0; pg < NP; ++pg) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const float z = I8 ? this->s0[rb] : 0.f;
          sp[pg][rb] = f32x4{z, z, z, z};
        }
#pragma unroll
        for (int ks = 0; ks < Base::KS; ++ks) {
          const Op8 ka = this->k_operand(page(cur_base, pg), ks);
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            sp[pg][rb] = Base::mfma32(ka, this->qB[rb][ks], sp[pg][rb]);
        }
      }
      if constexpr (I8) {
#pragma unroll
        for (int pg = 0; pg < NP; ++pg) {
          const char* sc = page(cur_base, pg) + 2 * Gm::PAGE;
          kwp[pg] = ld64(sc + 8 * c);
          vwp[pg] = ld64(sc + 32 + 8 * c);
        }
      }
    }
    if constexpr (kSteady && !I8) {
      constexpr int kDs = 0x100, kMfma = 0x008;      // scheduling-group masks: LDS reads, MFMAs
      __builtin_amdgcn_sched_group_barrier(kDs, kReadsAhead, 0);
#pragma unroll
      for (int i = 0; i < kPhaseReads - kReadsAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kDs, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kMfma, kPhaseMfma - (kPhaseReads - kReadsAhead), 0);
    }
  }

  // Softmax of the group whose first page is a (pages a .. a + NP - 1; those
  // at or past npages are copies, masked).
  template <bool EDGE>
  __device__ __forceinline__ void softmax_phase(int a, int npages) {
    constexpr int NV = 4 * NP;            // values per row block and lane
    if constexpr (I8) {
      // y = s * k_scale - m in one fma against the running maximum; the
      // exact maxima only when some row's reference moves
      float y[NRB][NV];
      bool move = false;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float t = -INFINITY;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int pg = j >> 2, i = j & 3;
          const int pos = (a + pg) * kPage + 4 * c + i;
          const float v = fmaf(sp[pg][rb][i], f16x2_half(kwp[pg][i >> 1], i & 1), -m[rb]);
          y[rb][j] = (!EDGE || (a + pg < npages && this->visible(pos, rb))) ? v : -INFINITY;
          t = fmaxf(t, y[rb][j]);
        }
        move |= xrow32_max(xrow16_max(t)) > kLazy;
      }
      if (__ballot(move)) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          float x[NV], t = -INFINITY;
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            const int pg = j >> 2, i = j & 3;
            const int pos = (a + pg) * kPage + 4 * c + i;
            const float v = sp[pg][rb][i] * f16x2_half(kwp[pg][i >> 1], i & 1);
            x[j] = (!EDGE || (a + pg < npages && this->visible(pos, rb))) ? v : -INFINITY;
            t = fmaxf(t, x[j]);
          }
          const float xm = xrow32_max(xrow16_max(t));
          const float mn = (xm > m[rb] + kLazy) ? xm : m[rb];
          const float alpha = __builtin_amdgcn_exp2f(m[rb] - mn);
          m[rb] = mn;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sacc[rb][i] *= alpha;
            lsum[rb][i] *= alpha;
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[rb][db][i] *= alpha;
          }
#pragma unroll
          for (int j = 0; j < NV; ++j) y[rb][j] = x[j] - mn;
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        // V scales of the lane's tokens as fp16 pairs, in k-slot order
        uint32_t vs[4] = {vwp[2 * u][0], vwp[2 * u][1], vwp[2 * u + 1][0], vwp[2 * u + 1][1]};
        if constexpr (EDGE) {
#pragma unroll
          for (int h = 0; h < 4; ++h) {    // garbage rows (scale may be NaN) weigh zero
            const int p0 = (a + 2 * u + (h >> 1)) * kPage + 4 * c + 2 * (h & 1);
            vs[h] &= (p0 < valid_end ? 0x0000ffffu : 0u) | (p0 + 1 < valid_end ? 0xffff0000u : 0u);
          }
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            pe[u][rb][h] = pack_f16x2(__builtin_amdgcn_exp2f(y[rb][8 * u + 2 * h]),
                                      __builtin_amdgcn_exp2f(y[rb][8 * u + 2 * h + 1]));
            pw[u][rb][h] = mul_f16x2(pe[u][rb][h], vs[h]);
          }
        }
      }
    } else {
      // masked unscaled scores, maxima scaled once per row, one fma per weight
      float x[NRB][NV], mx[NRB];
      bool move = false;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float t = -INFINITY;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int pg = j >> 2, i = j & 3;
          const int pos = (a + pg) * kPage + 4 * c + i;
          x[rb][j] = (!EDGE || (a + pg < npages && this->visible(pos, rb))) ? sp[pg][rb][i]
                                                                               : -INFINITY;
          t = fmaxf(t, x[rb][j]);
        }
        mx[rb] = xrow32_max(xrow16_max(t)) * scale_log2;
        move |= mx[rb] > m[rb] + kLazy;
      }
      if (__ballot(move)) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const float mn = (mx[rb] > m[rb] + kLazy) ? mx[rb] : m[rb];
          const float alpha = __builtin_amdgcn_exp2f(m[rb] - mn);
          m[rb] = mn;
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[rb][i] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[rb][db][i] *= alpha;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
          for (int h = 0; h < 4; ++h)
            pw[u][rb][h] = pack_bf16x2(
                __builtin_amdgcn_exp2f(fmaf(x[rb][8 * u + 2 * h], scale_log2, -m[rb])),
                __builtin_amdgcn_exp2f(fmaf(x[rb][8 * u + 2 * h + 1], scale_log2, -m[rb])));
        }
      }
    }
  }
};

// ============================================================================
// cross-workgroup merge of a pair split over several workgroups
// ============================================================================

// Floor quotients through one double division each (a 64-bit integer
// division is a long dependent sequence, on the path to the first page copy):
// with N < 2^31 and W <= 4096 the numerators stay below 2^43, exact in a
// double, and a quotient that is not an integer lies at least 1/W (resp.
// 1/N) from one while the rounding error stays below 2^-22, so truncating
// the correctly rounded quotient gives the exact floor.
__device__ __forceinline__ int64_t range_start(int w, int64_t N, int W) {
  return int64_t(double(int64_t(w) * N) / double(W));
}
// the workgroup (logical index) whose range holds global page x
__device__ __forceinline__ int wg_of(int64_t x, int64_t N, int W) {
  return int(double((x + 1) * W - 1) / double(N));
}
// Partial slot of workgroup w (range start g0) in the pair starting at
// pair_begin: its first slot when the pair starts inside its range.
__device__ __forceinline__ int slot_of(int w, int64_t g0, int64_t pair_begin) {
  return (max(g0, pair_begin) == g0) ? 2 * w : 2 * w + 1;
}

// Folds one partial state (m, l, o) into a running one (M, L, O).  Every merge
// of partials goes through this one sequence of operations (fixed fma forms),
// in segment order, so the result does not depend on which workgroup merges.
__device__ __forceinline__ void combine_partial(float& M, float& L, f32x4& O, float m, float l,
                                                const f32x4& o) {
  const float Mn = fmaxf(M, m);
  const float fa = exp2f(M - Mn), fb = exp2f(m - Mn);
  L = fmaf(fa, L, fb * l);
#pragma unroll
  for (int i = 0; i < 4; ++i) O[i] = fmaf(fa, O[i], fb * o[i]);
  M = Mn;
}

// Non-empty page ranges (segments) of the pair spanning workgroups wf .. wl.
__device__ __forceinline__ bool range_nonempty(int w, int64_t N, int W) {
  return N >= W || range_start(w + 1, N, W) > range_start(w, N, W);
}
__device__ __forceinline__ int pair_slot(int w, int wf, int first_slot) {
  return w == wf ? first_slot : 2 * w;
}
__device__ __forceinline__ int pair_segments(int wf, int wl, int64_t N, int W) {
  if (N >= W) return wl - wf + 1;
  int n = 0;
  for (int x = wf; x <= wl; ++x) n += range_start(x + 1, N, W) > range_start(x, N, W);
  return n;
}

template <int D, int NT>
__device__ __forceinline__ void merge_pair(const AttnParams& p, const Seg& sg, int64_t pb, int64_t pend,
                           int64_t N) {
  // Each thread merges up to kItems (row, 4-column) items; the loads of one
  // slot for all of them are issued together, so the merge costs one
  // device-scope load latency per slot instead of one per item and slot.
  constexpr int kItems = 4;
  const int wf = wg_of(pb, N, p.W), wl = wg_of(pend - 1, N, p.W);
  const int items = sg.R * (D / 4);
  for (int base = 0; base < items; base += kItems * NT) {
    float M[kItems], L[kItems];
    f32x4 O[kItems];
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
      M[u] = kNegBig;
      L[u] = 0.f;
      O[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // two slots per round (a pair usually spans two workgroups)
    for (int w0 = wf; w0 <= wl; w0 += 2) {
      float ms[2][kItems], ls[2][kItems];
      f32x4 os[2][kItems];
      bool use[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int w = w0 + h;
        use[h] = w <= wl && range_start(w + 1, N, p.W) > range_start(w, N, p.W);   // non-empty
        const int wu = use[h] ? w : w0;
        float* sb = slot_base<D>(p, slot_of(wu, range_start(wu, N, p.W), pb));
        const auto rs = slot_rsrc(sb, p.slot_rows * (D + 2) * 4);
#pragma unroll
        for (int u = 0; u < kItems; ++u) {
          const int it = base + u * NT + threadIdx.x;
          const int r = min(it, items - 1) / (D / 4), d4 = min(it, items - 1) % (D / 4);
          if (use[h]) {
            ms[h][u] = ld_dev1(rs, (p.slot_rows * D + r) * 4);
            ls[h][u] = ld_dev1(rs, (p.slot_rows * (D + 1) + r) * 4);
            os[h][u] = ld_dev4(rs, (r * D + 4 * d4) * 4);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (!use[h]) continue;
#pragma unroll
        for (int u = 0; u < kItems; ++u) combine_partial(M[u], L[u], O[u], ms[h][u], ls[h][u], os[h][u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
      const int it = base + u * NT + threadIdx.x;
      if (it >= items) continue;
      const int r = it / (D / 4), d4 = it % (D / 4);
      const float inv = 1.f / L[u];
      f32x4 o = O[u];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= inv;
      store_out4(p, out_row(p, sg, r) * D + 4 * d4, o);
    }
  }
}

// Merge of a pair split over several workgroups, fused with the last one's
// wave merge.  Each workgroup of the pair, once its waves' states are in LDS,
// counts its arrival (device-scope counter) and merges its waves' states into
// registers; every workgroup but the last to arrive writes its partial and
// then counts it as published (second counter).  The last to arrive waits for
// the others' publications -- they have all arrived, so they are running and
// publish without waiting on anything -- and folds every segment of the pair
// in segment order, its own from registers and the others from their slots,
// through combine_partial: the same operations whichever workgroup is last.
// Saves the last workgroup a write, a fence and a reload of its own partial.
// Split pairs of at most 32 query rows (one pass over the pages) take this
// path.  The last workgroup resets the arrival counter (every workgroup of
// the pair has arrived) and takes the others' publications back off the
// publication counter.  Its wait is bounded (p.wait_polls polls); if it
// gives up, the pair's output rows are written as NaN (never a fold of
// partials that may not be there), bit 0 of the status word is set, and the
// publications still to come bring the counter back to zero before the
// kernel ends, so the workspace stays reusable.
constexpr int kSpinLimit = 1 << 22;

// The current segment's pair: global page range [pb, pend) and total pages N,
// kept in LDS (not in registers through the page loop).
__device__ __forceinline__ int64_t* pair_info() {
  __shared__ int64_t s_pair[3];
  return s_pair;
}
// This workgroup's logical index: consecutive ranges go to one XCD.
__device__ __forceinline__ int logical_wg(int W) {
  const int hw = blockIdx.x;
  return (W % 8 == 0) ? (hw % 8) * (W / 8) + hw / 8 : hw;
}
// Whether this workgroup is the last of the current pair to arrive.
__device__ __forceinline__ int& pair_last() {
  __shared__ int s_last;
  return s_last;
}
// Whether the last workgroup's wait for the others' partials succeeded.
__device__ __forceinline__ int& pair_ok() {
  __shared__ int s_ok;
  return s_ok;
}
// The current pair's arrival counter and its number of segments.
__device__ __forceinline__ int32_t* pair_arrivals(const AttnParams& p) {
  return p.counters + wg_of(pair_info()[0], pair_info()[2], p.W);
}
__device__ __forceinline__ int pair_nseg(const AttnParams& p) {
  const int64_t pb = pair_info()[0], pend = pair_info()[1], N = pair_info()[2];
  return pair_segments(wg_of(pb, N, p.W), wg_of(pend - 1, N, p.W), N, p.W);
}

template <class St, int D, int NT>
__device__ __forceinline__ void merge_fused(const AttnParams& p, const Seg& sg, const float* mrg,
                                            int stride) {
  constexpr int RW = St::SLOT_ROWS;
  constexpr int ITEMS = RW * (D / 4);
  constexpr int J = (ITEMS + NT - 1) / NT;
  const int tid = merge_tid<true>();
  const int64_t pb = pair_info()[0], pend = pair_info()[1], N = pair_info()[2];
  const int wf = wg_of(pb, N, p.W), wl = wg_of(pend - 1, N, p.W);
  int32_t* published = p.counters + kMaxWorkgroups + wf;
  float M[J], L[J];
  f32x4 O[J];
  St::merge_prepare(mrg, NT / kWave, stride, tid);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int it = tid + j * NT;
    if (it < ITEMS) St::merge_any(mrg, NT / kWave, stride, it % RW, it / RW, M[j], L[j], O[j]);
  }
  if (!pair_last()) {                  // set before the barrier that ended the stream
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int it = tid + j * NT;
      if (it < ITEMS && it % RW < sg.R) St::write_partial(p, sg, it % RW, it / RW, M[j], L[j], O[j]);
    }
    // the partial's stores are complete at device scope before the count
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(published, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (tid == 0) {
    const int others = pair_segments(wf, wl, N, p.W) - 1;
    int ok = 0;
    for (int n = 0; n < p.wait_polls; ++n) {
      if (__hip_atomic_load(published, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= others) {
        ok = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (!ok) __hip_atomic_fetch_or(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pair_ok() = ok;
  }
  __syncthreads();
  const bool ok = pair_ok() != 0;
  float Mc[J], Lc[J];
  f32x4 Oc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    Mc[j] = kNegBig;
    Lc[j] = 0.f;
    Oc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // segments in order, up to kBatch at a time: every load of a batch is
  // issued before its partials are folded in, so a batch costs one latency
  constexpr int kBatch = 3;
  const int self = logical_wg(p.W);
  const int first_slot = slot_of(wf, range_start(wf, N, p.W), pb);
  int w = ok ? wf : wl + 1;            // after a give-up nothing is read
  while (w <= wl) {
    int ws[kBatch];
    int n = 0;
    for (; w <= wl && n < kBatch; ++w)
      if (range_nonempty(w, N, p.W)) ws[n++] = w;   // non-empty
    float ms[kBatch][J], ls[kBatch][J];
    f32x4 os[kBatch][J];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (k >= n || ws[k] == self) continue;
      float* sb = slot_base<D>(p, pair_slot(ws[k], wf, first_slot));
      const auto rs = slot_rsrc(sb, p.slot_rows * (D + 2) * 4);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int it = min(tid + j * NT, ITEMS - 1);
        const int r = min(it % RW, sg.R - 1), d4 = it / RW;
        ms[k][j] = ld_dev1(rs, (p.slot_rows * D + r) * 4);
        ls[k][j] = ld_dev1(rs, (p.slot_rows * (D + 1) + r) * 4);
        os[k][j] = ld_dev4(rs, (r * D + 4 * d4) * 4);
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (k >= n) continue;
      const bool own = ws[k] == self;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (own) combine_partial(Mc[j], Lc[j], Oc[j], M[j], L[j], O[j]);
        else combine_partial(Mc[j], Lc[j], Oc[j], ms[k][j], ls[k][j], os[k][j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int it = tid + j * NT;
    if (it >= ITEMS || it % RW >= sg.R) continue;
    const float inv = 1.f / Lc[j];
    f32x4 o = Oc[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = ok ? o[i] * inv : __builtin_nanf("");
    store_out4(p, out_row(p, sg, it % RW) * D + 4 * (it / RW), o);
  }
  if (tid == 0) {
    const int others = pair_segments(wf, wl, N, p.W) - 1;
    __hip_atomic_store(p.counters + wf, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(published, -others, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One pass over the segment's pages for rows r0.. of the pair: stream, then
// merge the NW waves through LDS.  MFMA steps: each wave's ring region is
// large enough for its state, so a wave stores its state there as soon as its
// own pages are done, and one round spread over all threads merges them;
// VALU steps merge pairwise through the idle ring and wave 0 writes the output
// rows or the partial slot.
// Bytes of a wave's LDS region in the split-step pass: its ring, then (the
// same bytes) its final state.
template <typename KV, int D, int NW, class St>
__device__ __forceinline__ constexpr int wave_region() {
  constexpr int GR = Geo<KV, D, NW>::RING;
  constexpr int SB = St::SLOT_F * 4;
  return GR > SB ? GR : SB;
}

// issued: the first steps' page copies of this pass are already in flight.
template <typename KV, int D, int NW, class St>
__device__ __forceinline__ void pass(const AttnParams& p, const Seg& sg, int r0, St& st,
                                     char* ring_all, bool issued = false) {
  const int wave = wave_id();
  constexpr int GR = Geo<KV, D, NW>::RING;
  if constexpr (St::kSplit) {
    constexpr int WR = wave_region<KV, D, NW, St>();  // this wave's ring, then its state
    char* mine = ring_all + wave * WR;
    run_pages<KV, D, NW>(p, sg, mine, st, issued);
    // a split pair's arrival is counted as soon as wave 0's pages are done, so
    // the counter's round trip overlaps the other waves' last pages
    int old = 0;
    if (sg.fuse && threadIdx.x == 0)
      old = __hip_atomic_fetch_add(pair_arrivals(p), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st.finish();
    st.store(reinterpret_cast<float*>(mine));        // no other wave touches this region
    if (sg.fuse && threadIdx.x == 0) pair_last() = (old == pair_nseg(p) - 1);
    __syncthreads();
    const float* mrg = reinterpret_cast<const float*>(ring_all);
    if (sg.fuse) merge_fused<St, D, NW * kWave>(p, sg, mrg, WR / 4);
    else St::merge_write(p, sg, r0, mrg, NW, WR / 4);
    __syncthreads();
  } else {
    run_pages<KV, D, NW>(p, sg, ring_all + wave * GR, st);
    st.finish();
    __syncthreads();                                  // every wave is off the ring
    float* mrg = reinterpret_cast<float*>(ring_all);
    constexpr int SLOT = St::SLOT_F;
#pragma unroll
    for (int half = NW / 2; half >= 1; half /= 2) {
      if (wave >= half && wave < 2 * half) st.store(mrg + (wave - half) * SLOT);
      __syncthreads();
      if (wave < half) st.combine(mrg + wave * SLOT);
      __syncthreads();
    }
    if (wave == 0) st.write(p, sg, r0);
    __syncthreads();
  }
}

// ============================================================================
// kernel
// ============================================================================

template <typename KV, int D, bool MF>
struct AttnLds {
  static constexpr int NW = (MF && sizeof(KV) == 1) ? kWavesInt8 : kWavesValu;
  static constexpr int NT = NW * kWave;
  // MFMA: each wave's region holds its ring, then its state (two row blocks
  // at most); VALU: the wave merge reuses the ring (NW/2 slots of the state)
  static constexpr int GR = Geo<KV, D, NW>::RING;
  static constexpr int SB = MF ? 4 * (2 * (D / 16) * kWave * 4 + 4 * kWave) : 0;
  static constexpr int RING = NW * (GR > SB ? GR : SB);
  static constexpr int MERGE = MF ? 0 : (NW / 2) * 4 * (kValuRows * D * 2 + 64);
  static constexpr int RING_ALLOC = RING > MERGE ? RING : MERGE;
  // VALU passes stage their query rows and per-wave probabilities in LDS
  static constexpr int QS = MF ? 4 : kValuRows * 2 * (D / 2 + 4);   // dwords (fp32 layout, the larger)
  static constexpr int PS = MF ? 16 : kValuRows * 32 * 4;           // bytes per wave
};

// The MFMA and VALU variants are separate kernels, so that each gets its own
// register allocation.
template <typename KV, int D, bool MF>
__device__ __forceinline__ void process_segment(const AttnParams& p, const Seg& sg, char* ring,
                                                uint32_t* qs, char* ps_all) {
  if constexpr (MF) {
    // The first pass's first page copies go out before its step is set up
    // (query loads, row masks): that set-up is on the path to the first data,
    // and the prologue as a whole is on the kernel's (a 2 us wait at entry
    // lengthened the 7B MHA kernel by 1.2-1.7 us).
    constexpr int NW = AttnLds<KV, D, MF>::NW;
    {
      constexpr int S = Geo<KV, D, NW>::S;
      const int wave = wave_id();
      const int npair = (sg.pe - sg.pa + 1) >> 1;
      int q[S];
#pragma unroll
      for (int i = 0; i < S; ++i) q[i] = wave + NW * i < npair ? wave + NW * i : -1;
      char* mine = ring + wave * (sg.R > 16 ? wave_region<KV, D, NW, MfmaStep<KV, D, 2>>()
                                            : wave_region<KV, D, NW, MfmaStep<KV, D, 1>>());
      issue_first_steps<KV, D, NW>(p, sg, mine, wave, q);
    }
    for (int r0 = 0; r0 < sg.R; r0 += kMfmaRows) {
      if (sg.R - r0 > 16) {
        MfmaStep<KV, D, 2> st(p, sg, r0);
        pass<KV, D, NW>(p, sg, r0, st, ring, r0 == 0);
      } else {
        MfmaStep<KV, D, 1> st(p, sg, r0);
        pass<KV, D, NW>(p, sg, r0, st, ring, r0 == 0);
      }
    }
    return;
  }
  // fp32 caches take at most 8 rows per pass (16 fp32 rows exceed the register file)
  constexpr bool F32 = sizeof(KV) == 4;
  constexpr int kRows = F32 ? 8 : kValuRows;
  char* ps = ps_all + wave_id() * AttnLds<KV, D, MF>::PS;
  for (int r0 = 0; r0 < sg.R; r0 += kRows) {
    valu_stage_q<D, F32>(p, sg, r0, qs);
    __syncthreads();
    const int rn = sg.R - r0;
    if (rn <= 4) {
      ValuStep<KV, D, 4> st(p, sg, r0, qs, ps);
      pass<KV, D, AttnLds<KV, D, MF>::NW>(p, sg, r0, st, ring);
    } else if (F32 || rn <= 8) {
      ValuStep<KV, D, 8> st(p, sg, r0, qs, ps);
      pass<KV, D, AttnLds<KV, D, MF>::NW>(p, sg, r0, st, ring);
    } else {
      ValuStep<KV, D, 16> st(p, sg, r0, qs, ps);
      pass<KV, D, AttnLds<KV, D, MF>::NW>(p, sg, r0, st, ring);
    }
  }
}

// ============================================================================
// append of the new rows, fused into the verification pass
// ============================================================================
//
// HeteroReason, workflow Phase 3: the target appends the speculated rows to
// the cache and verifies them in the same pass.  A new row is written by the
// wave that will copy its page (wave w copies units -- pairs of pages --
// w, w + NW, ... of each segment), before that wave issues any page copy, with
// the same conversion (and INT8 rule) as sva_kv_append; no other wave and no
// other workgroup reads that row of that kv head in this call.  A wave's
// memory operations complete in issue order and every step waits for its own
// copies, so the stores are complete before any copy issued after the
// wave's first wait -- every copy but the first S steps of the first
// segment.  A wave that holds new rows in those steps waits for its stores
// before issuing them; the others start streaming at once.  16 lanes per
// row; out-of-contract positions (past the block table, invalid page ids)
// are skipped as the append does.  Returns whether the wave must wait.
template <typename KV, typename Src, int D, int NW>
__device__ __forceinline__ bool append_wave_rows(const AttnParams& p, int64_t g0, int64_t g1,
                                                 int b, int64_t sb) {
  // g0, g1, sb: cost coordinates (see pair_pos)
  constexpr int N = D / kRowLanes;
  constexpr int S_RING = Geo<KV, D, NW>::S;          // steps issued before the first wait
  const int wave = wave_id();
  const int group = lane_id() / kRowLanes, sub = lane_id() % kRowLanes;
  bool early = false;
  bool first = true;
  SeqInfo si = seq_info(p, b);
  int64_t cur = g0;
  while (cur < g1) {
    while (cur >= sb + seq_cost(p, si)) {             // next sequence with pages
      sb += seq_cost(p, si);
      ++b;
      si = seq_info(p, b);
    }
    const PairPos pp = pair_pos(p, cur, sb, si.np, g1);
    const int g = pp.g, pa = pp.pa, pe = pp.pe;
    const int64_t se = min(g1, pp.bend);
    // positions S .. S+k-1 whose page lies in [pa, pe), 4 per pass (one per
    // 16-lane group), each written by the owner of its unit
    const int lo = max(si.S, pa * kPage), hi = min(si.S + si.k, pe * kPage);
    for (int pos0 = lo; pos0 < hi; pos0 += kWave / kRowLanes) {
      const int pos = pos0 + group;                     // uniform per 16-lane row
      const int lp = pos / kPage;
      const int u = (lp - pa) >> 1;
      if (pos >= hi || u % NW != wave || lp >= p.max_pages) continue;
      const int page = p.block_table[int64_t(b) * p.max_pages + lp];
      if (page < 0 || page >= p.num_pages) continue;
      if (first && u / NW < S_RING) early = true;
      // (kv_shift is 0 here: a call whose pairs split the query heads appends
      // in a launch of its own, so that no row is written by two workgroups)
      const int64_t src_row = int64_t(si.q0 + (pos - si.S)) * p.Hkv + g;
      const int64_t dst_row = (int64_t(page) * p.Hkv + g) * kPage + (pos % kPage);
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        float v[N];
        Chunk<Src, N>::load(static_cast<const Src*>(which ? p.v_new : p.k_new) + src_row * D + sub * N,
                            v);
        if constexpr (sizeof(KV) == 1) {
          int8_t c[N];
          const uint16_t s16 = quant_row<N>(v, c);
          store_codes<N>(static_cast<int8_t*>(const_cast<void*>(which ? p.v : p.k)) + dst_row * D + sub * N,
                         c);
          if (sub == 0) const_cast<uint16_t*>(which ? p.v_scale : p.k_scale)[dst_row] = s16;
        } else {
          Chunk<KV, N>::store(static_cast<KV*>(const_cast<void*>(which ? p.v : p.k)) + dst_row * D + sub * N,
                              v);
        }
      }
    }
    if (pe > pa) first = false;
    cur = se;
  }
  return __ballot(early) != 0;
}

template <typename KV, int D, bool MF>
__global__ __launch_bounds__((AttnLds<KV, D, MF>::NT), 1) void verify_attn_kernel(AttnParams p) {
  using L = AttnLds<KV, D, MF>;
  constexpr int NT = L::NT;
  __shared__ __attribute__((aligned(1024))) char s_ring[L::RING_ALLOC];
  __shared__ __attribute__((aligned(16))) uint32_t s_q[L::QS];
  __shared__ __attribute__((aligned(16))) char s_ps[L::NW * L::PS];
  __shared__ int32_t s_scan[NT];
  __shared__ int32_t s_info[4];
  __shared__ int32_t s_seq[4];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int B = p.B;

  // ---- pages per sequence: each thread sums a contiguous chunk of sequences
  // (the first kSeqCache of them stay in registers for the search below)
  constexpr int kSeqCache = 4;
  const int per = (B + NT - 1) / NT;
  int tot = 0;
  SeqInfo cache[kSeqCache];
#pragma unroll
  for (int e = 0; e < kSeqCache; ++e) {
    const int b = tid * per + e;
    cache[e] = SeqInfo{0, 0, 0, 0};
    if (e < per && b < B) {
      cache[e] = seq_info(p, b);
      tot += int(seq_cost(p, cache[e]));
    }
  }
  for (int e = kSeqCache; e < per; ++e) {
    const int b = tid * per + e;
    if (b < B) tot += int(seq_cost(p, seq_info(p, b)));
  }
  s_scan[tid] = tot;
  __syncthreads();
  if (tid < kWave) {                                  // exclusive scan of the chunk sums
    constexpr int PER_LANE = NT / kWave;
    int run = 0;
    for (int i = 0; i < PER_LANE; ++i) {
      const int v = s_scan[tid * PER_LANE + i];
      s_scan[tid * PER_LANE + i] = run;
      run += v;
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o, kWave);
      if (tid >= o) incl += u;
    }
    const int excl = incl - run;
    for (int i = 0; i < PER_LANE; ++i) s_scan[tid * PER_LANE + i] += excl;
    if (tid == kWave - 1) s_info[0] = incl;           // total cost N
  }
  __syncthreads();
  const int64_t N = s_info[0];
  if (N == 0) return;

  // ---- this workgroup's range (cost coordinates); consecutive ranges go to one XCD
  const int w = logical_wg(p.W);
  const int64_t g0 = range_start(w, N, p.W), g1 = range_start(w + 1, N, p.W);
  if (g0 >= g1) return;

  // the sequence holding page g0, the first page of that sequence and its
  // SeqInfo (from the registers above when cached: no second load)
  {
    const int base = s_scan[tid];
    if (tot > 0 && base <= g0 && g0 < base + tot) {
      int run = base;
      for (int e = 0; e < per; ++e) {
        const int b = tid * per + e;
        SeqInfo si_e = cache[0];
#pragma unroll
        for (int c = 1; c < kSeqCache; ++c)
          if (e == c) si_e = cache[c];
        if (e >= kSeqCache) si_e = seq_info(p, b);
        const int n = int(seq_cost(p, si_e));
        if (g0 < run + n) {
          s_info[1] = b;
          s_info[2] = run;
          s_seq[0] = si_e.S;
          s_seq[1] = si_e.k;
          s_seq[2] = si_e.q0;
          s_seq[3] = si_e.np;
          break;
        }
        run += n;
      }
    }
  }
  __syncthreads();
  int b = s_info[1];
  int64_t sb = s_info[2];
  if (p.k_new) {                                      // this wave's new rows first
    const bool early = p.src_f32 ? append_wave_rows<KV, float, D, L::NW>(p, g0, g1, b, sb)
                                 : append_wave_rows<KV, uint16_t, D, L::NW>(p, g0, g1, b, sb);
    if (early) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  SeqInfo si{s_seq[0], s_seq[1], s_seq[2], s_seq[3]};

  int64_t cur = g0;
  while (cur < g1) {
    while (cur >= sb + seq_cost(p, si)) {             // next sequence with pages
      sb += seq_cost(p, si);
      ++b;
      si = seq_info(p, b);
    }
    const PairPos pp = pair_pos(p, cur, sb, si.np, g1);
    const int64_t pb = pp.pb, pend = pp.pend;
    const int64_t se = min(g1, pp.bend);
    if (pp.pe <= pp.pa) {               // only the pair's fixed cost lies in the range
      cur = se;
      continue;
    }
    Seg sg;
    sg.b = b;
    sg.g = pp.g;
    sg.pa = pp.pa;
    sg.pe = pp.pe;
    sg.S = si.S;
    sg.k = si.k;
    sg.q0 = si.q0;
    sg.np = si.np;
    sg.R = si.k * p.G;
    sg.full = pp.pa == 0 && pp.pe == si.np;
    sg.slot = slot_of(w, g0, pb);
    sg.fuse = MF && !sg.full && sg.R <= kMfmaRows;
    if (sg.fuse && tid == 0) {          // read after the barriers of the pass
      pair_info()[0] = pb;
      pair_info()[1] = pend;
      pair_info()[2] = N;
    }

    process_segment<KV, D, MF>(p, sg, s_ring, s_q, s_ps);

    if (!sg.full && !sg.fuse) {
      // every thread's partial stores are complete at device scope before the
      // barrier, so the increment below is ordered after all of them
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) {
        const int wf = wg_of(pb, N, p.W), wlast = wg_of(pend - 1, N, p.W);
        int nseg = 0;
        for (int x = wf; x <= wlast; ++x)
          nseg += range_start(x + 1, N, p.W) > range_start(x, N, p.W);
        const int old = __hip_atomic_fetch_add(p.counters + wf, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        s_flag = (old == nseg - 1);
      }
      __syncthreads();
      if (s_flag) {      // the last workgroup of the pair: all partials are visible
        merge_pair<D, NT>(p, sg, pb, pend, N);
        if (tid == 0)
          __hip_atomic_store(p.counters + wg_of(pb, N, p.W), 0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    }
    cur = se;
  }
}

// ============================================================================
// row-block kernel: many query rows per pair (long speculated steps)
// ============================================================================
//
// Step-level verification scores a whole speculated step -- tens to hundreds
// of drafts -- in one pass ("HeteroReason": the PRM verifies a complete step
// in a single parallel pass).  With k*G query rows per (sequence, kv head) far
// above 32, splitting the keys over waves (the kernel above) would re-stream
// the pages once per 32 rows.  Here a workgroup owns a block of up to 256
// query rows of one pair (a pair's rows spread evenly over its blocks, in
// whole waves), each of its 8 waves 32 of them, and all eight share every
// page.  A group is NU units of two pages (bf16: 2, INT8: 1, whose operands
// take more registers); groups stream through a workgroup ring of 4 to 8
// slots, copied several groups ahead by 2 NU waves of the second half (one
// page each, at the start of their softmax phase, the phase with time to
// spare), or by the last wave alone when it holds no rows.
// A wave never merges with another.  While the blocks fill the device,
// nothing is split over workgroups and no workspace is used; fewer blocks (a
// few long steps) are cut into key slices, each writing its rows' partial
// state to the workspace, and a second launch (verify_rows_merge_kernel)
// folds them.  Keys are streamed up to the block's last row's position; the
// causal (or tree) mask applies on the pages holding drafts.
//
// Each SIMD holds one wave of each half of the workgroup (waves w and w + 4).
// Per group a wave runs a product phase (P.V of the previous group, S^T of
// this one: matrix cores and LDS reads) and a softmax phase (vector ALU only).
// The two halves run them half a group apart, separated by workgroup barriers:
//
//   phase 2w     first half: products of group w     second half: softmax of group w-1
//   phase 2w+1   first half: softmax of group w      second half: products of group w
//
// so on every SIMD one wave's matrix products run beside the other wave's
// softmax, and the product phases run at raised wave priority (without it:
// 5 % slower).  Two units per group halve the barriers per page against one
// (7B reward-model shape: 144 us against 155).  Slot of group u: read in
// phases 2u .. 2u+3, refilled (group u + NS) from phase 2u+4 on.
// Iterations whose units need no mask run in a loop of their own: with both
// kinds in one loop body the compiler keeps two copies of the accumulators at
// the join and spills the query operands.

constexpr int kRowWaves = 8;                       // two waves per SIMD
constexpr int kRowHalf = kRowWaves / 2;
constexpr int kRowBlock = kRowWaves * kMfmaRows;   // 256 query rows per workgroup
constexpr int kRowMergeThreads = 256;
constexpr int kMinSliceGroups = 4;                  // groups of pages per key slice, at least
constexpr size_t kCounterBytes = size_t(2 * kMaxWorkgroups) * 4 + 256;
// A key slice's partial state of one row block: unnormalised O [256][D], then
// the running maxima [256] and the weight sums [256] (fp32).
template <int D>
constexpr int kRowSlotFloats = kRowBlock * (D + 2);

template <typename KV, int D>
struct RowsLds {
  using Gm = Geo<KV, D, kWavesValu>;
  static constexpr int NU = sizeof(KV) == 1 ? 1 : 2;  // units per group
  static constexpr int NP = 2 * NU;                   // pages per group
  static constexpr int UNIT = NP * Gm::SLOT;          // K, V (and scales) of a group
  static constexpr int NS_RAW = (128 * 1024) / UNIT;
  static constexpr int NS = NS_RAW > 8 ? 8 : NS_RAW;  // groups held in the ring
  static constexpr int RING = NS * UNIT;
  static_assert(NS >= 4, "ring too small");
  static_assert((NS - 3) * Gm::P <= 63, "vmcnt range");
};

// Row blocks of sequence b: Hkv * ceil(k_b * G / 256), times nseg key slices.
__device__ __forceinline__ int row_blocks(const AttnParams& p, const SeqInfo& si, int nseg) {
  return si.k > 0 ? p.Hkv * ((si.k * p.G + kRowBlock - 1) / kRowBlock) * nseg : 0;
}

// The blocks of the batch lie sequence after sequence.  rows_scan: NT threads
// each count the blocks of a contiguous chunk of sequences (returned) and
// their exclusive prefix sums go to s_scan; the total to s_info[0].
template <int NT>
__device__ __forceinline__ int rows_scan(const AttnParams& p, int nseg, int32_t* s_scan,
                                         int32_t* s_info) {
  const int tid = threadIdx.x;
  const int per = (p.B + NT - 1) / NT;
  int tot = 0;
  for (int e = 0; e < per; ++e) {
    const int b = tid * per + e;
    if (b < p.B) tot += row_blocks(p, seq_info(p, b), nseg);
  }
  s_scan[tid] = tot;
  __syncthreads();
  if (tid < kWave) {
    constexpr int PER_LANE = NT / kWave;
    int run = 0;
    for (int i = 0; i < PER_LANE; ++i) {
      const int v = s_scan[tid * PER_LANE + i];
      s_scan[tid * PER_LANE + i] = run;
      run += v;
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o, kWave);
      if (tid >= o) incl += u;
    }
    const int excl = incl - run;
    for (int i = 0; i < PER_LANE; ++i) s_scan[tid * PER_LANE + i] += excl;
    if (tid == kWave - 1) s_info[0] = incl;
  }
  __syncthreads();
  return tot;
}
// rows_find: block w (< the total) lies in sequence s_info[1], which starts at
// block s_info[3]; s_info[2] = w - s_info[3].  Ends with a barrier.
template <int NT>
__device__ __forceinline__ void rows_find(const AttnParams& p, int nseg, int w, int tot,
                                          const int32_t* s_scan, int32_t* s_info) {
  const int tid = threadIdx.x;
  const int per = (p.B + NT - 1) / NT;
  const int base = s_scan[tid];
  if (tot > 0 && base <= w && w < base + tot) {
    int run = base;
    for (int e = 0; e < per; ++e) {
      const int b = tid * per + e;
      const int n = row_blocks(p, seq_info(p, b), nseg);
      if (w < run + n) {
        s_info[1] = b;
        s_info[2] = w - run;
        s_info[3] = run;
        break;
      }
      run += n;
    }
  }
  __syncthreads();
}

// Wait until at most n (<= MAXN) later units of P copies each are in flight.
template <int P, int MAXN>
__device__ __forceinline__ void wait_units(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      wait_vm<MAXN * P>();
      return;
    }
    wait_units<P, MAXN - 1>(n);
  } else {
    wait_vm<0>();
  }
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// kTree: the call carries tree masks (at most 32 drafts, mask form); causal
// calls keep draft indices (any number of drafts).
template <typename KV, int D, bool kTree>
__global__ __launch_bounds__(kRowWaves * kWave, 1)
void verify_attn_rows_kernel(AttnParams p) {
  using Gm = Geo<KV, D, kWavesValu>;
  using L = RowsLds<KV, D>;
  constexpr int NS = L::NS;
  constexpr int NT = kRowWaves * kWave;
  __shared__ __attribute__((aligned(1024))) char s_ring[L::RING];
  __shared__ int32_t s_scan[NT];
  __shared__ int32_t s_info[4];
  const int nseg = p.rows_nseg;

  // ---- this workgroup's block: exclusive scan of the per-sequence counts
  const int tot = rows_scan<NT>(p, nseg, s_scan, s_info);
  const int total = s_info[0];
  // Workgroups are dispatched to the 8 XCDs in turn (blockIdx.x % 8), one per
  // CU here (the ring takes most of the LDS): XCD x takes blocks
  // x * ceil(total / 8) onwards, so every XCD holds an equal share and
  // consecutive blocks (the row blocks of one pair, which read the same
  // pages) share an L2.  The grid is a multiple of 8 at least total.
  const int hw = blockIdx.x;
  const int per_xcd = (total + 7) / 8;
  const int j = hw / 8;
  const int w = (hw % 8) * per_xcd + j;
  if (j >= per_xcd || w >= total) return;
  rows_find<NT>(p, nseg, w, tot, s_scan, s_info);
  const int b = s_info[1];
  const SeqInfo si = seq_info(p, b);
  const int nblk = (si.k * p.G + kRowBlock - 1) / kRowBlock;
  // within the sequence: kv head, then key slice, then row block, so that the
  // row blocks of one slice (which read the same pages) are neighbours
  const int x = s_info[2];
  const int seg = (x / nblk) % nseg, rbk = x % nblk;
  Seg sg;
  sg.b = b;
  sg.g = x / (nblk * nseg);
  sg.S = si.S;
  sg.k = si.k;
  sg.q0 = si.q0;
  sg.np = si.np;
  sg.R = si.k * p.G;
  sg.pa = 0;
  sg.full = true;
  sg.slot = 0;
  // The pair's rows are spread evenly over its blocks (whole waves of 32):
  // blocks that stream at one pace keep each page in L2 for the others (a
  // half-empty last block ran ahead of its pair and the rest fetched its
  // pages again: 1.8x the pages' bytes from memory).
  const int rpb = ((sg.R + nblk - 1) / nblk + kMfmaRows - 1) / kMfmaRows * kMfmaRows;
  const int r0 = rbk * rpb;
  const int r_end = min(sg.R, r0 + rpb);
  const int last_row = r_end - 1;
  // keys up to the last row's position: pages 0 .. npages-1, in groups of NP
  constexpr int NP = L::NP;
  const int npages = min(si.np, (si.S + last_row / p.G) / kPage + 1);
  sg.pe = npages;
  // Key slice seg: groups [ua, ua + nunits) of the pair's groups cut into
  // nseg equal ranges (the same cut for every row block of the pair), up to
  // this block's last group; loop indices below count from ua.
  const int npages_pair = min(si.np, (si.S + (sg.R - 1) / p.G) / kPage + 1);
  const int nunits_pair = (npages_pair + NP - 1) / NP;
  const int ua = seg * nunits_pair / nseg;
  const int nunits = max(0, min((seg + 1) * nunits_pair / nseg, (npages + NP - 1) / NP) - ua);
  // groups below u_plain hold committed context only: no masks
  const int u_plain = max(0, min(nunits, si.S / (NP * kPage) - ua));
  const int wave = wave_id();
  const int half = wave / kRowHalf;
  const int rw = r0 + kMfmaRows * wave;            // this wave's first row
  const bool active = rw < r_end;                   // wave-uniform
  PhaseStep<KV, D, L::NU, !kTree> st(p, sg, rw);
  // The copies: a block with a wave that holds no rows (the last wave) has
  // that wave copy every page of each group, off the phases' critical paths
  // (7B-shaped long step: 2.5 % faster in A/B runs); otherwise NP waves of the
  // second half copy one page each at the start of their softmax phase.  The
  // idle copier's waits leave NS - 3 whole groups in flight, within the 6-bit
  // vmcnt (issue past 63 outstanding copies stalls until one lands).
  constexpr bool kIdleOk = (NS - 3) * NP * Gm::P <= 63;
  const bool idle_copier = kIdleOk && r_end - r0 < kRowWaves * kMfmaRows;
  const int cw = wave - kRowHalf;
  const bool copier = idle_copier ? wave == kRowWaves - 1 : (cw >= 0 && cw < NP);
  auto slot = [&](int u) __attribute__((always_inline)) -> const char* { return s_ring + (u % NS) * L::UNIT; };
  // pages past the end copy the last page (unused)
  auto issue = [&](int u) __attribute__((always_inline)) {          // wave j: page NP (ua + u) + j
    if (u >= nunits) return;
    if (idle_copier) {
      int ids[NP];
#pragma unroll
      for (int j = 0; j < NP; ++j) ids[j] = page_id(p, b, min(NP * (ua + u) + j, npages - 1));
#pragma unroll
      for (int j = 0; j < NP; ++j)
        dma_page<KV, D, false>(p, ids[j], sg.g, s_ring + (u % NS) * L::UNIT + j * Gm::SLOT);
      return;
    }
    const int pg = min(NP * (ua + u) + cw, npages - 1);
    dma_page<KV, D, false>(p, page_id(p, b, pg), sg.g,
                           s_ring + (u % NS) * L::UNIT + cw * Gm::SLOT);
  };
  // copies of group u landed (this wave's), later groups may still fly
  auto wait_unit = [&](int u) __attribute__((always_inline)) {
    if (!copier || u >= nunits) return;
    if constexpr (kIdleOk) {
      if (idle_copier) {
        wait_units<Gm::P * NP, NS - 3>(min(NS - 3, nunits - 1 - u));
        return;
      }
    }
    wait_units<Gm::P, NS - 3>(min(NS - 3, nunits - 1 - u));
  };
  if (copier) {
    for (int u = 0; u < NS - 2; ++u) issue(u);
  }
  st.ready();
  wait_unit(0);
  block_barrier();

  auto products = [&](int u, auto edge) __attribute__((always_inline)) {           // P.V of group u-1, S^T of group u
    constexpr bool EDGE = decltype(edge)::value;
    __builtin_amdgcn_s_setprio(1);
    st.template mma_phase<EDGE>(slot(u + NS - 1), NP * (ua + u - 1), u > 0, slot(u), u < nunits);
    __builtin_amdgcn_s_setprio(0);
  };
  // groups 1 .. u_plain - 1: both groups of the phase exist and need no masks
  auto products_steady = [&](int u) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    st.template mma_phase<false, true>(slot(u + NS - 1), NP * (ua + u - 1), true, slot(u), true);
    __builtin_amdgcn_s_setprio(0);
  };
  auto softmax = [&](int u, auto edge) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge)::value;
    st.template softmax_phase<EDGE>(NP * (ua + u), npages);
  };
  // iteration w: phases 2w and 2w+1.  The copies of group w + NS - 2 go into
  // the slot that group w - 2 left in phase 2w - 1, and group w + 1 has
  // landed before the barrier that ends phase 2w + 1.  Each half runs a loop
  // of its own, so each loop body is straight-line code; both halves pass the
  // same number of barriers.  A wave without rows only keeps the barriers
  // (and its copies).
  if (half == 0) {
    auto iteration = [&](int w, auto edge) __attribute__((always_inline)) {
      if (active) products(w, edge);
      block_barrier();
      if (active && w < nunits) softmax(w, edge);
      block_barrier();
    };
    int it = 0;
    if (u_plain > 0) iteration(it++, std::false_type{});
    for (; it < u_plain; ++it) {
      if (active) products_steady(it);
      block_barrier();
      if (active) softmax(it, std::false_type{});
      block_barrier();
    }
    for (; it <= nunits; ++it) iteration(it, std::true_type{});
  } else {
    auto iteration = [&](int w, auto edge) __attribute__((always_inline)) {
      if (copier) issue(w + NS - 2);
      if (active && w > 0) softmax(w - 1, edge);
      block_barrier();
      if (active) products(w, edge);
      wait_unit(w + 1);
      block_barrier();
    };
    int it = 0;
    if (u_plain > 0) iteration(it++, std::false_type{});
    for (; it < u_plain; ++it) {
      if (copier) issue(it + NS - 2);
      if (active) softmax(it - 1, std::false_type{});
      block_barrier();
      if (active) products_steady(it);
      wait_unit(it + 1);
      block_barrier();
    }
    for (; it <= nunits; ++it) iteration(it, std::true_type{});
  }
  if (active) {
    st.finish();
    if (nseg == 1) {
      st.write_rows(p, sg, rw);
    } else {                                     // this slice's partial state
      const int slot = ((s_info[3] / nseg) + sg.g * nblk + rbk) * nseg + seg;
      st.write_partial(p.partials + int64_t(slot) * kRowSlotFloats<D>, rw - r0, kRowBlock);
    }
  }
}

// Key slices of the row blocks: workgroup w folds the nseg partial states of
// rows kMergeRows (w % kMergeParts) .. + kMergeRows of row block
// w / kMergeParts, slice by slice in key order (the same operations whatever
// the grid), and writes them normalised.  One (row, 4-column) item per
// thread; the states of 8 slices are loaded together before they are folded,
// so an item costs a memory round trip per 8 slices.
template <int D>
__global__ __launch_bounds__(kRowMergeThreads) void verify_rows_merge_kernel(AttnParams p) {
  constexpr int NT = kRowMergeThreads;
  constexpr int kMergeRows = NT / (D / 4);
  constexpr int kMergeParts = kRowBlock / kMergeRows;
  constexpr int kBatch = 8;
  __shared__ int32_t s_scan[NT];
  __shared__ int32_t s_info[4];
  const int nseg = p.rows_nseg;
  const int tot = rows_scan<NT>(p, 1, s_scan, s_info);
  const int w = blockIdx.x / kMergeParts;
  if (w >= s_info[0]) return;
  rows_find<NT>(p, 1, w, tot, s_scan, s_info);
  const int b = s_info[1];
  const SeqInfo si = seq_info(p, b);
  const int nblk = (si.k * p.G + kRowBlock - 1) / kRowBlock;
  Seg sg;
  sg.b = b;
  sg.g = s_info[2] / nblk;
  sg.q0 = si.q0;
  sg.R = si.k * p.G;
  const int rpb = ((sg.R + nblk - 1) / nblk + kMfmaRows - 1) / kMfmaRows * kMfmaRows;
  const int r0 = (s_info[2] % nblk) * rpb;
  const int rows = min(sg.R, r0 + rpb) - r0;
  const int r = (blockIdx.x % kMergeParts) * kMergeRows + int(threadIdx.x) / (D / 4);
  const int d4 = int(threadIdx.x) % (D / 4);
  if (r >= rows) return;
  const float* base = p.partials + int64_t(w) * nseg * kRowSlotFloats<D>;
  float M = kNegBig, L = 0.f;
  f32x4 O{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nseg; s0 += kBatch) {
    float ms[kBatch], ls[kBatch];
    f32x4 os[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float* sl = base + int64_t(min(s0 + i, nseg - 1)) * kRowSlotFloats<D>;
      ms[i] = sl[kRowBlock * D + r];
      ls[i] = sl[kRowBlock * (D + 1) + r];
      os[i] = *reinterpret_cast<const f32x4*>(sl + r * D + 4 * d4);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (s0 + i < nseg) combine_partial(M, L, O, ms[i], ls[i], os[i]);
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int i = 0; i < 4; ++i) O[i] *= inv;
  store_out4(p, out_row(p, sg, r0 + r) * D + 4 * d4, O);
}

// ============================================================================
// host side
// ============================================================================

AttnPlan plan_verify_attn(const sva_batch* batch, const sva_paged_kv* kv, int Hq, int num_cus,
                          const sva_verify_opts* opts, size_t max_bytes) {
  AttnPlan pl;
  const int G = Hq / kv->Hkv;
  // Row-block kernel: when a pair has more query rows than the split kernel
  // handles in one pass and the blocks alone fill the device, or (bf16
  // caches) the query-head split below cannot bring a pair to one pass, or
  // the split kernel cannot take the shape at all.  MFMA path only.  For
  // bf16, pairs of 33-128 rows that the split kernel streams once per pass
  // run faster as row blocks, cut into key slices where they are few (G = 7,
  // k = 8, 64 pairs: 62.3 -> 42.9 us; G = 7, k = 16, 16 pairs: 71.2 ->
  // 25.3 us; G = 8, k = 8, 192 pairs: 145.5 -> 85.8 us); the INT8 row-block
  // kernel is slower there (G = 7, k = 8, 64 pairs: 45.0 -> 53.9 us).
  const bool mfma_ok = kv->kv_dtype != SVA_F32 && !(opts && opts->path == 1);
  const int64_t rows = int64_t(std::max(batch->max_q, 1)) * G;
  const int64_t blocks_ub =
      int64_t(kv->Hkv) * ((int64_t(batch->total_q) * G + kRowBlock - 1) / kRowBlock + batch->B);
  const int64_t kv_pairs = int64_t(batch->B) * kv->Hkv;
  int one_pass_split = 1;             // the query-head split that fits one pass
  while (rows / one_pass_split > kMfmaRows && G % (2 * one_pass_split) == 0 &&
         kv_pairs * 2 * one_pass_split <= num_cus)
    one_pass_split *= 2;
  const bool split_passes = rows / one_pass_split > kMfmaRows;
  pl.rows_kernel = mfma_ok && (batch->max_q > kMaxDraftsSplit || rows > kMaxRowsSplit ||
                               (rows > kMfmaRows && blocks_ub >= num_cus) ||
                               (split_passes && kv->kv_dtype == SVA_BF16));
  const int64_t pages_per_seq =
      std::min<int64_t>(kv->max_pages_per_seq, (int64_t(batch->max_len) + kPage - 1) / kPage);
  // Key slices for the row-block kernel when its blocks leave CUs idle (a few
  // long steps): about one block per CU, each slice at least kMinSliceGroups
  // groups of pages, and the partial states within max_bytes.
  pl.rows_nseg = 1;
  const size_t row_slot_bytes = size_t(kRowBlock) * (kv->d + 2) * sizeof(float);
  if (pl.rows_kernel) {
    const int group_pages = kv->kv_dtype == SVA_INT8 ? 2 : 4;
    const int64_t groups = (std::max<int64_t>(pages_per_seq, 1) + group_pages - 1) / group_pages;
    int64_t ns = std::min<int64_t>(num_cus / std::max<int64_t>(blocks_ub, 1),
                                   groups / kMinSliceGroups);
    const size_t avail = max_bytes > kCounterBytes ? max_bytes - kCounterBytes : 0;
    ns = std::min<int64_t>(ns, int64_t(avail / (row_slot_bytes * size_t(std::max<int64_t>(blocks_ub, 1)))));
    if (ns > 1) pl.rows_nseg = int(std::min<int64_t>(ns, 64));
  }
  // a multiple of 8 (the kernel spreads its blocks evenly over the 8 XCDs)
  pl.rows_grid = int(std::min<int64_t>((blocks_ub * pl.rows_nseg + 7) / 8 * 8, 0x7ffffff8));
  // merge: kRowBlock / (kRowMergeThreads / (d / 4)) workgroups per row block
  pl.rows_merge_grid = int(std::min<int64_t>(
      blocks_ub * (kRowBlock / (kRowMergeThreads / (kv->d / 4))), 0x7fffffff));
  // Query heads split over workgroups: a kv head's G query heads form
  // kv_split pairs of G / kv_split, streamed by neighbouring workgroups of
  // one XCD that read the same pages at about the same time (the later read
  // mostly hits L2).  First until a pair's rows fit one 32-row pass: a pair
  // with more rows is otherwise streamed once per pass (8B-shaped GQA, G = 8,
  // k = 8, 64 pairs: 63.5 -> 40.3 us; 128 pairs: 100.6 -> 61.8 us; k = 16,
  // G = 8, 16 pairs, in four: 134.6 -> 56.1 us).  Then once more for few pairs (at
  // most one per 8 CUs) of 32 rows: every pair is cut into half as many
  // segments for the same grid and each merge folds half as many rows (one
  // GPU's TP-8 share of the 70B INT8 shape: 27.1 -> 21.0 us; 4 sequences of
  // 8192 tokens, G = 8, k = 4: bf16 39.4 -> 36.0 us, INT8 30.0 -> 25.8 us).
  // Not for pairs of 16 rows or fewer (half an MFMA block per part: 4 x 8192
  // tokens, G = 4, k = 4 took 32.7 -> 35 us), nor for many pairs of 32 rows
  // (the whole 70B INT8 shape: the later reads missed L2, 1.36x the KV bytes,
  // and the call was slower), nor beyond one pair per CU: the parts of a kv
  // head must stream at the same time, on different workgroups, for L2 to
  // serve the later reads.
  pl.kv_split = 1;
  if (!pl.rows_kernel && mfma_ok) {
    pl.kv_split = one_pass_split;
    if (rows / pl.kv_split >= kMfmaRows && G % (2 * pl.kv_split) == 0 &&
        kv_pairs * pl.kv_split * 8 <= num_cus)
      pl.kv_split *= 2;
  }
  const int64_t npairs = kv_pairs * pl.kv_split;
  const int64_t pages_ub = npairs * std::max<int64_t>(pages_per_seq, 1);
  int W = 0;
  if (opts && opts->num_workgroups > 0) {
    W = std::min(opts->num_workgroups, kMaxWorkgroups);
  } else {
    const int64_t want = (pages_ub + 15) / 16;     // at least 4 pages per wave
    // Splitting a pair over one more workgroup shortens its stream by a share
    // of its pages but adds a partial to its merge, which one workgroup reads
    // after the others finish; a partial costs about as much as streaming 8
    // pages, so the time is lowest near sqrt(pages per pair / 8) segments.
    const int64_t seg_cap =
        std::max<int64_t>(2, int64_t(std::sqrt(double(std::max<int64_t>(pages_per_seq, 1)) / 8.0) + 0.5));
    W = int(std::min<int64_t>(std::min<int64_t>(std::min(std::max(num_cus, 1), kMaxWorkgroups),
                                                std::max<int64_t>(want, 1)),
                              npairs * seg_cap));
  }
  pl.num_wg = W;
  // fixed cost of a segment in pages: about kSegCostBytes of streaming
  const int page_bytes = 2 * kPage * kv->d * (kv->kv_dtype == SVA_F32 ? 4 : kv->kv_dtype == SVA_BF16 ? 2 : 1) +
                         (kv->kv_dtype == SVA_INT8 ? 4 * kPage : 0);
  pl.seg_cost = int((kSegCostBytes + page_bytes / 2) / page_bytes);
  pl.wait_polls = !opts || opts->wait_polls == 0 ? kSpinLimit : std::max(opts->wait_polls, 0);
  pl.slot_rows = std::max(batch->max_q, 1) * (G / pl.kv_split);
  // arrival and publication counters, then the status word (256 bytes keep
  // the partial slots aligned)
  pl.counter_bytes = kCounterBytes;
  pl.slot_bytes = size_t(2) * W * pl.slot_rows * (kv->d + 2) * sizeof(float);
  pl.total_bytes = pl.counter_bytes + pl.slot_bytes;
  if (pl.rows_kernel) {                 // the key slices' partial states, if any
    pl.num_wg = 0;
    pl.slot_bytes = pl.rows_nseg > 1 ? row_slot_bytes * size_t(blocks_ub) * pl.rows_nseg : 0;
    pl.total_bytes = pl.counter_bytes + pl.slot_bytes;
  }
  return pl;
}

template <typename KV, int D>
static hipError_t attn_rows_launch(const AttnParams& p, int grid, int merge_grid, hipStream_t st) {
  if (p.draft_mask)
    hipLaunchKernelGGL((verify_attn_rows_kernel<KV, D, true>), dim3(grid), dim3(kRowWaves * kWave),
                       0, st, p);
  else
    hipLaunchKernelGGL((verify_attn_rows_kernel<KV, D, false>), dim3(grid), dim3(kRowWaves * kWave),
                       0, st, p);
  if (p.rows_nseg > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((verify_rows_merge_kernel<D>), dim3(merge_grid), dim3(kRowMergeThreads), 0,
                       st, p);
  }
  return hipGetLastError();
}

template <typename KV, int D>
static hipError_t attn_launch(const AttnParams& p, bool mfma, hipStream_t st) {
  if constexpr (sizeof(KV) == 4) {
    hipLaunchKernelGGL((verify_attn_kernel<KV, D, false>), dim3(p.W),
                       dim3(AttnLds<KV, D, false>::NT), 0, st, p);
  } else if (mfma) {
    hipLaunchKernelGGL((verify_attn_kernel<KV, D, true>), dim3(p.W),
                       dim3(AttnLds<KV, D, true>::NT), 0, st, p);
  } else {
    hipLaunchKernelGGL((verify_attn_kernel<KV, D, false>), dim3(p.W),
                       dim3(AttnLds<KV, D, false>::NT), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_verify_attn(const sva_batch* batch, const void* q, int q_dtype, int Hq,
                              const sva_paged_kv* kv, const uint32_t* draft_mask,
                              float softmax_scale, void* out, int out_dtype, int path,
                              const AttnPlan& plan, void* workspace, hipStream_t st,
                              const void* k_new, const void* v_new, int src_dtype) {
  AttnParams p;
  p.q = q;
  p.draft_mask = draft_mask;
  p.k_new = k_new;
  p.v_new = v_new;
  p.src_f32 = src_dtype == SVA_F32;
  p.k = kv->k;
  p.v = kv->v;
  p.k_scale = static_cast<const uint16_t*>(kv->k_scale);
  p.v_scale = static_cast<const uint16_t*>(kv->v_scale);
  p.block_table = kv->block_table;
  p.ctx_lens = batch->ctx_lens;
  p.cu_q = batch->cu_q;
  p.out = out;
  p.counters = static_cast<int32_t*>(workspace);
  p.status = p.counters + 2 * kMaxWorkgroups;
  p.wait_polls = plan.wait_polls;
  p.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.counter_bytes);
  p.scale_log2 = softmax_scale * kLog2e;
  p.q_f32 = q_dtype == SVA_F32;
  p.out_f32 = out_dtype == SVA_F32;
  p.B = batch->B;
  p.T = batch->total_q;
  p.Hq = Hq;
  p.Hkv = kv->Hkv * plan.kv_split;
  p.G = Hq / kv->Hkv / plan.kv_split;
  p.kv_shift = __builtin_ctz(unsigned(plan.kv_split));
  p.rows_nseg = plan.rows_nseg;
  p.num_pages = kv->num_pages;
  p.max_pages = kv->max_pages_per_seq;
  p.max_q = batch->max_q;
  p.slot_rows = plan.slot_rows;
  p.W = plan.num_wg;
  p.seg_cost = plan.seg_cost;
  const bool mfma = path != 1;         // fp32 caches always take the VALU kernel
  if (plan.rows_kernel) {
    // the row-block kernel reads a pair's draft pages from several
    // workgroups: the new rows are appended by their own launch first
    if (k_new) {
      const hipError_t e = launch_kv_append(batch, k_new, v_new, src_dtype, kv, st);
      if (e != hipSuccess) return e;
    }
    if (plan.rows_grid <= 0) return hipSuccess;
    const int mg = plan.rows_merge_grid;
    if (kv->kv_dtype == SVA_BF16)
      return kv->d == 64 ? attn_rows_launch<uint16_t, 64>(p, plan.rows_grid, mg, st)
                         : attn_rows_launch<uint16_t, 128>(p, plan.rows_grid, mg, st);
    return kv->d == 64 ? attn_rows_launch<int8_t, 64>(p, plan.rows_grid, mg, st)
                       : attn_rows_launch<int8_t, 128>(p, plan.rows_grid, mg, st);
  }
  if (k_new && plan.kv_split > 1) {     // every part of a kv head reads its new rows
    const hipError_t e = launch_kv_append(batch, k_new, v_new, src_dtype, kv, st);
    if (e != hipSuccess) return e;
    p.k_new = p.v_new = nullptr;
  }
  if (kv->kv_dtype == SVA_F32)
    return kv->d == 64 ? attn_launch<float, 64>(p, false, st) : attn_launch<float, 128>(p, false, st);
  if (kv->kv_dtype == SVA_BF16)
    return kv->d == 64 ? attn_launch<uint16_t, 64>(p, mfma, st)
                       : attn_launch<uint16_t, 128>(p, mfma, st);
  return kv->d == 64 ? attn_launch<int8_t, 64>(p, mfma, st) : attn_launch<int8_t, 128>(p, mfma, st);
}

}  // namespace sva
