// Internal launchers of libspecverify (host side).  Each enqueues kernels on
// `st` and returns the launch status; argument checking happens in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

namespace sva {

hipError_t launch_kv_quant_int8(const void* x, int src_dtype, int64_t rows, int d, int8_t* codes,
                                uint16_t* scales, hipStream_t st);

hipError_t launch_kv_append(const sva_batch* batch, const void* k_new, const void* v_new,
                            int src_dtype, const sva_paged_kv* kv, hipStream_t st);

// Verification attention.  `num_wg` is the grid size; the workspace holds the
// completion counters and the status word, followed by the partial-result
// slots.
struct AttnPlan {
  bool rows_kernel;     // row-block kernel (many query rows per pair); no workspace
  int rows_grid;        // its grid (an upper bound on the row blocks times rows_nseg)
  int rows_nseg;        // key slices per row block (> 1: a merge launch follows)
  int rows_merge_grid;  // the merge's grid (an upper bound on the row blocks)
  int num_wg;
  int wait_polls;       // bound on a split pair's wait for the others' partials
  int seg_cost;         // fixed cost of a segment, in pages, for the work split
  int slot_rows;
  int kv_split;         // pairs per kv head (its query heads split over workgroups)
  size_t counter_bytes;
  size_t slot_bytes;
  size_t total_bytes;
};
// max_bytes: the workspace the plan may need at most (the row-block kernel's
// key slices are limited to it).
AttnPlan plan_verify_attn(const sva_batch* batch, const sva_paged_kv* kv, int Hq, int num_cus,
                          const sva_verify_opts* opts, size_t max_bytes = size_t(1) << 30);
// draft_mask: [T] tree attention masks (bit j: draft j of the sequence is
// visible), or NULL for causal drafts.
// k_new / v_new (may be NULL): [T, Hkv, d] rows of src_dtype appended to the
// cache at positions S_b .. S_b+k_b-1 before the attention reads them.
hipError_t launch_verify_attn(const sva_batch* batch, const void* q, int q_dtype, int Hq,
                              const sva_paged_kv* kv, const uint32_t* draft_mask,
                              float softmax_scale, void* out, int out_dtype, int path,
                              const AttnPlan& plan, void* workspace, hipStream_t st,
                              const void* k_new = nullptr, const void* v_new = nullptr,
                              int src_dtype = 0);

// Acceptance: chunked argmax then a per-sequence scan.
struct AcceptPlan {
  int rows;
  int chunks;
  int chunk_len;
  size_t total_bytes;
};
AcceptPlan plan_accept(const sva_batch* batch, int V);
// Kernel 1 of acceptance: per (row, chunk) the 64-bit key of the chunk's
// first maximum (order-preserving float bits above the complemented index).
hipError_t launch_argmax_keys(const float* logits, int V, const AcceptPlan& plan, uint64_t* keys,
                              hipStream_t st);
hipError_t launch_accept_prefix(const sva_batch* batch, const float* logits, int V,
                                const int32_t* draft_ids, int32_t* argmax_ids, int32_t* accept_len,
                                int32_t* next_token, const AcceptPlan& plan, void* workspace,
                                hipStream_t st);

// Token trees: ancestor masks, greedy tree acceptance, and the move of the
// accepted branch's K/V rows to the positions right after the context.
hipError_t launch_tree_masks(const sva_batch* batch, const int32_t* parents, uint32_t* masks,
                             hipStream_t st);
hipError_t launch_accept_tree(const sva_batch* batch, const float* logits, int V,
                              const int32_t* draft_ids, const int32_t* parents,
                              int32_t* argmax_ids, int32_t* accept_len, int32_t* next_token,
                              int32_t* accept_path, const AcceptPlan& plan, void* workspace,
                              hipStream_t st);
hipError_t launch_kv_commit_path(const sva_batch* batch, const int32_t* accept_len,
                                 const int32_t* accept_path, const sva_paged_kv* kv,
                                 hipStream_t st);

// Stochastic acceptance: row statistics over chunks, per-sequence decisions,
// then inverse-CDF sampling of one row per sequence.  Workspace: chunk
// statistics of every target and draft row, one record per sequence, and the
// per-chunk weight sums of the sampled rows.
struct SamplePlan {
  int stat_rows;
  int chunks;                               // row statistics: chunks per row
  int chunk_len;
  int s_chunks;                             // sampled rows: chunks per row
  int s_len;
  int per;                                  // elements per thread range of a sampled chunk
  size_t stats_off, rec_off, sums_off, parts_off;
  size_t total_bytes;
};
SamplePlan plan_sample(const sva_batch* batch, int V);
hipError_t launch_accept_stochastic(const sva_batch* batch, const float* target_logits,
                                    const float* draft_logits, int V, float temperature,
                                    const int32_t* draft_ids, const float* u_accept,
                                    const float* u_sample, int32_t* accept_len,
                                    int32_t* next_token, const SamplePlan& plan, void* workspace,
                                    hipStream_t st);

// Streaming-read probe: `bytes` (a multiple of 1 KB) read once by `num_wg`
// workgroups, into registers (mode 0) or through global -> LDS copies (mode
// 1); sink [num_wg * 4] receives one word per wave.
hipError_t launch_stream_read_probe(const void* buf, size_t bytes, int mode, int num_wg,
                                    uint32_t* sink, hipStream_t st);

// Pages of the speculative history: return pages wholly past the valid
// lengths to a free list; give unassigned pages below S_b + k_b pages from it.
hipError_t launch_kv_reclaim_pages(int B, const int32_t* valid_lens, int32_t* block_table,
                                   int max_pages, int32_t* free_list, int32_t* free_count,
                                   int capacity, hipStream_t st);
hipError_t launch_kv_alloc_pages(const sva_batch* batch, int32_t* block_table, int max_pages,
                                 const int32_t* free_list, int32_t* free_count, int capacity,
                                 hipStream_t st);

// KVMU pointer triplets: one thread per sequence applies its mode.
hipError_t launch_kvmu(int B, const int32_t* mode, int uniform_mode, const int32_t* arg,
                       int32_t* state, int32_t* ctx_lens, hipStream_t st);

}  // namespace sva
