/*
 * specverify.h -- C ABI of libspecverify.so, the MI355X (gfx950) hot path of
 * speculative-decoding verification.
 *
 * The target model scores the k_b draft tokens of every sequence in one pass
 * ("Decoding Speculative Decoding from First Principles", section
 * "Speculating to get sequence parallelism during decode").  Four operations:
 *
 *   sva_kv_quant_int8     INT8 KV rows with one fp16 absmax scale per row
 *   sva_kv_append         write the k_b new K/V rows into the paged cache
 *   sva_spec_verify_attn  causal multi-query attention of the k_b drafts
 *   sva_accept_prefix     greedy longest-prefix acceptance over the logits
 *
 * and, on the same conventions, a fused form of two of them
 * (sva_spec_verify_attn_append) and the token-tree, stochastic-acceptance
 * and KV-pointer calls further below.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as device memory are HIP device pointers owned by the
 *   caller.  Structs are read on the host during the call and not kept.
 * - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *   Every call only enqueues work on that stream and returns; nothing is
 *   synchronised.  The library allocates no memory.
 * - Host-checkable argument errors return SVA_ERR_INVALID_ARG or
 *   SVA_ERR_UNSUPPORTED before anything is enqueued, and nothing is written.
 *   A failed launch returns SVA_ERR_HIP.  sva_last_error() gives the detail
 *   (thread-local, valid until the next call on the same thread).
 * - Values that live in device memory (ctx_lens, cu_q, block-table entries)
 *   are preconditions.  Kernels clamp out-of-contract values so that they
 *   never access memory outside the buffers described here, but the results
 *   for such inputs are unspecified.
 * - Only gfx950 devices are supported (SVA_ERR_UNSUPPORTED otherwise).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVA_OK = 0,
  SVA_ERR_INVALID_ARG = 1,
  SVA_ERR_UNSUPPORTED = 2,
  SVA_ERR_HIP = 3
} sva_status;

typedef enum { SVA_F32 = 0, SVA_BF16 = 1, SVA_F16 = 2, SVA_INT8 = 3 } sva_dtype;

/* Paged KV cache of ONE attention layer.  Pages hold `page_size` (= 16)
 * consecutive token positions of one sequence; a page of one kv head is
 * contiguous ("CXL-SpecKV", memory hierarchy section: the pool is organised in
 * 4 KB pages -- 16 tokens x 128 values x 2 bytes).
 *   k, v                 [num_pages, Hkv, page_size, d] of kv_dtype
 *                        (SVA_F32, SVA_BF16 or SVA_INT8 codes)
 *   k_scale, v_scale     [num_pages, Hkv, page_size] fp16 bit patterns; only for
 *                        SVA_INT8 (value = code * scale), NULL otherwise
 *   block_table          [B, max_pages_per_seq] int32: physical page of each
 *                        logical page of each sequence; -1 marks unused entries
 * Logical position p of sequence b lives at page block_table[b][p / 16],
 * slot p % 16. */
typedef struct {
  void *k;
  void *v;
  void *k_scale;
  void *v_scale;
  const int32_t *block_table;
  int32_t num_pages;
  int32_t page_size;
  int32_t Hkv;
  int32_t d;
  int32_t max_pages_per_seq;
  int32_t kv_dtype;
} sva_paged_kv;

/* One verification batch of B sequences ("HeteroReason", KVMU description,
 * Fig. 7: ctx_lens[b] is the validated pointer; ctx_lens[b] + k_b the
 * speculation frontier while the drafts are verified).
 *   ctx_lens   [B] device int32: committed rows S_b, EXCLUDING this step's drafts
 *   cu_q       [B+1] device int32: prefix sums of k_b (cu_q[0] = 0); k_b may be 0
 *   total_q    host copy of cu_q[B] (T, the number of draft rows)
 *   max_q      host upper bound on every k_b (1..16; 1..1024 for sva_kv_append
 *              and sva_spec_verify_attn, 1..32 for sva_spec_verify_attn_tree)
 *   max_len    host upper bound on every S_b + k_b */
typedef struct {
  int32_t B;
  const int32_t *ctx_lens;
  const int32_t *cu_q;
  int32_t total_q;
  int32_t max_q;
  int32_t max_len;
} sva_batch;

/* Optional tuning for sva_spec_verify_attn; pass NULL for the defaults.
 *   path            0: default -- MFMA for bf16 and INT8 caches, VALU for fp32
 *                   1: VALU for every sequence     2: MFMA (same as 0)
 *   num_workgroups  0: chosen from the device and batch; otherwise the grid size,
 *                   1 .. 4096 (must equal the value used for the workspace size
 *                   query)
 *   wait_polls      bound on the one wait inside the kernel: the workgroup that
 *                   finishes a pair split over several workgroups waits for the
 *                   others' partial results (they are all running by then, so
 *                   the wait takes microseconds).  0: the default, 2^22 polls;
 *                   n > 0: at most n polls; negative: no poll at all, so every
 *                   such wait gives up (a way to exercise the failure path).
 *                   A wait that gives up writes NaN to the rows of that pair and
 *                   sets bit 0 of the workspace status word (see
 *                   sva_spec_verify_attn); the workspace stays reusable.  Where
 *                   the planner splits a kv head's G query heads over 2 or 4
 *                   workgroups (pairs of more than 32 query rows, or few
 *                   pairs), a pair is that share of the heads, and so are its
 *                   NaN rows. */
typedef struct {
  int32_t path;
  int32_t num_workgroups;
  int32_t wait_polls;
} sva_verify_opts;

/* INT8 quantisation of `rows` rows of d values, one fp16 scale per row.
 * "CXL-SpecKV", Algorithm 2 (KV-Cache Compression), steps 3 and 5, and key
 * observation (4):  a = max|x|,  scale = fp16_rne(a / 127),
 * code = clamp(rne(fp32(x / scale)), -127, 127), codes 0 when scale == 0.
 *   x        device [rows, d] of src_dtype (SVA_F32 or SVA_BF16)
 *   codes    device [rows, d] int8 (written)
 *   scales   device [rows] fp16 bit patterns (written)
 *   d        64, 128 or 256
 * Inputs must be finite with max|x| <= 65504 * 127 (the scale must fit fp16). */
sva_status sva_kv_quant_int8(const void *x, int32_t src_dtype, int64_t rows, int32_t d,
                             int8_t *codes, uint16_t *scales, void *stream);

/* Append the k_b new K and V rows of every sequence at logical positions
 * S_b .. S_b + k_b - 1 ("HeteroReason", workflow Phase 3: the cache holds the
 * context plus the speculated rows; rows past the validated length are
 * invalid after a rejection).
 *   k_new, v_new   device [T, Hkv, d] of src_dtype (SVA_F32 or SVA_BF16),
 *                  rows ordered by cu_q
 *   kv             the cache; rows are stored as kv_dtype: F32 and BF16 caches
 *                  round to nearest-even, INT8 caches quantise each (token,
 *                  head) row exactly as sva_kv_quant_int8
 * Block-table entries for the written positions must be valid pages. */
sva_status sva_kv_append(const sva_batch *batch, const void *k_new, const void *v_new,
                         int32_t src_dtype, const sva_paged_kv *kv, void *stream);

/* Workspace bytes that sva_spec_verify_attn needs for this batch shape on the
 * current device (depends on B, Hkv, d, max_q, max_len, Hq and opts). */
size_t sva_verify_workspace_bytes(const sva_batch *batch, const sva_paged_kv *kv, int32_t Hq,
                                  const sva_verify_opts *opts);

/* Causal verification attention.  For sequence b, draft query i (position
 * S_b + i) and query head h (kv head g = h / G, G = Hq / Hkv):
 *   out[cu_q[b]+i][h] = sum_p softmax_p(scale * q . K_p) V_p,  p = 0 .. S_b + i
 * ("Decoding Speculative Decoding from First Principles": the target verifies
 * every draft in one prefill-style pass with causal masking; "CXL-SpecKV", key
 * observation (1): a token reads all earlier positions).  K/V rows of INT8
 * caches are code * scale.
 *   q           device [T, Hq, d] of q_dtype (SVA_F32 or SVA_BF16)
 *   out         device [T, Hq, d] of out_dtype (SVA_F32 or SVA_BF16), written
 *   workspace   device, >= sva_verify_workspace_bytes(...) bytes.  Its first
 *               32 KB hold completion counters (two per workgroup, for any grid
 *               size), the next 256 bytes a status word (int32 at byte 32768):
 *               all must be zero before the workspace is first used.  Every
 *               call leaves the counters all-zero again, so one workspace
 *               serves calls of any shape in stream order.  The status word is
 *               only ever set, never cleared, by the library: bit 0 means a
 *               wait gave up (see sva_verify_opts.wait_polls) and the rows of
 *               the pair concerned were written as NaN; the caller reads and
 *               clears it when it wants to know.  Calls that may run
 *               concurrently need distinct workspaces.
 * Supported: page_size 16, d in {64, 128}, Hq % Hkv == 0, B <= 4096, and
 * max_q <= 16 with max_q * (Hq / Hkv) <= 128 on every path; bf16 and INT8
 * caches on the MFMA path (the default) also take long speculated steps,
 * max_q <= 1024 ("HeteroReason": a process reward model verifies a whole
 * reasoning step in one parallel pass).  Pairs with many query rows (k_b * G
 * above 32, when their 256-row blocks fill the device, and always above 16
 * drafts or 128 rows) run on a row-block kernel that reads each page once per
 * block of 256 rows.  When those blocks are fewer than the CUs (a few long
 * steps), each block's keys are cut into slices streamed by separate
 * workgroups, whose partial states (256 * (d + 2) fp32 per block and slice)
 * the workspace holds and a second launch folds in key order; otherwise the
 * row-block kernel needs no more workspace than the counters.  SVA_F32
 * caches always take the VALU path (query rows past 16 are handled in further
 * passes over the pages). */
sva_status sva_spec_verify_attn(const sva_batch *batch, const void *q, int32_t q_dtype,
                                int32_t Hq, const sva_paged_kv *kv, float softmax_scale,
                                void *out, int32_t out_dtype, const sva_verify_opts *opts,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes that sva_accept_prefix needs for this batch and vocab. */
size_t sva_accept_workspace_bytes(const sva_batch *batch, int32_t V);

/* Greedy longest-prefix acceptance ("Decoding Speculative Decoding from First
 * Principles", section "Speculating to get sequence parallelism during
 * decode": reject at the first disagreement, keep the target's token; the last
 * row yields the +1 bonus token).
 *   logits      device [T + B, V] fp32; sequence b owns the k_b + 1 rows that
 *               start at cu_q[b] + b (row j scores the token after draft j-1)
 *   draft_ids   device [T] int32
 *   argmax_ids  device [T + B] int32 (written): first index of each row's
 *               maximum; a NaN counts as the maximum (first NaN wins);
 *               -0.0 equals +0.0
 *   accept_len  device [B] int32 (written): n_b = leading drafts equal to the
 *               target's tokens (0 .. k_b)
 *   next_token  device [B] int32 (written): the target's token at row n_b
 *   workspace   device, >= sva_accept_workspace_bytes(...) bytes, no
 *               initialisation needed
 * The step emits draft[0 .. n_b-1] followed by next_token[b]: n_b + 1 tokens.
 * Committing is the caller's: S_b += n_b + 1 once the bonus token's K/V row is
 * appended by the next step (or S_b += n_b before it). */
sva_status sva_accept_prefix(const sva_batch *batch, const float *logits, int32_t V,
                             const int32_t *draft_ids, int32_t *argmax_ids, int32_t *accept_len,
                             int32_t *next_token, void *workspace, size_t workspace_bytes,
                             void *stream);

/* ---- Token trees ------------------------------------------------------------
 * "Decoding Speculative Decoding from First Principles", section "Tree based
 * verification" (SpecInfer, EAGLE-2, DDTree): the drafter proposes a tree of
 * continuations, tree attention relates each draft only to its own lineage,
 * and the accepted continuation is the longest branch the target agrees with.
 * A tree of k_b <= 16 nodes is given per sequence as
 *   parents   device [T] int32, rows ordered by cu_q: the parent of node i is
 *             -1 (a child of the last committed token) or an earlier node
 *             0 .. i-1 (topological order); any other value is read as -1.
 * Node i's K/V row sits at position S_b + i (sva_kv_append writes it there).
 * A chain (parent i-1) is the causal case of the calls above. */

/* Ancestor masks: masks[cu_q[b] + i] gets bit j set when node j of sequence b
 * is node i or one of its ancestors (bits >= k_b are zero).  One call per
 * verification step; the masks serve every layer's attention call.
 *   masks   device [T] uint32 (written) */
sva_status sva_tree_masks(const sva_batch *batch, const int32_t *parents, uint32_t *masks,
                          void *stream);

/* Tree attention: sva_spec_verify_attn with the causal draft mask replaced by
 *   draft_mask  device [T] uint32: draft i of sequence b sees the committed
 *               positions 0 .. S_b - 1 and the drafts j < k_b whose bit j is
 *               set in draft_mask[cu_q[b] + i] (normally sva_tree_masks'
 *               output).  Every other argument, the workspace included, is as
 *               for sva_spec_verify_attn; a row that sees no key at all
 *               (S_b = 0 and an empty mask) has no defined output. */
sva_status sva_spec_verify_attn_tree(const sva_batch *batch, const void *q, int32_t q_dtype,
                                     int32_t Hq, const sva_paged_kv *kv,
                                     const uint32_t *draft_mask, float softmax_scale, void *out,
                                     int32_t out_dtype, const sva_verify_opts *opts,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* sva_spec_verify_attn for callers that cannot allocate -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc: the
 * same kernels and results, with the workspace taken from a static device
 * array of the library instead of an argument.  Every other argument is as
 * for sva_spec_verify_attn (causal drafts; no tree mask).
 *   - The array holds 16 MiB per device (allocated when the library's code is
 *     loaded on that device, held until the process ends).  A shape whose
 *     workspace (sva_verify_workspace_bytes) exceeds it returns
 *     SVA_ERR_UNSUPPORTED before anything is enqueued; at d = 128 and 256
 *     workgroups that is above 62 query rows per pair (k_b * G, or the share
 *     of it a pair keeps where the query heads are split over workgroups).
 *     Long speculated steps whose row blocks are cut into key slices take
 *     as many slices as the array holds (fewer than sva_spec_verify_attn may
 *     take), so they are never refused for it.
 *   - The first call on a device takes the array's address and enqueues one
 *     small kernel on `stream` that zeroes its counters; no call allocates
 *     memory.
 *   - Every call on a device shares that device's array, which keeps the last
 *     call's contents: calls that may overlap on one device (different streams
 *     or threads without ordering) race and give undefined results.
 *   - A wait that gives up writes NaN to the rows of its pair, as documented
 *     for sva_verify_opts.wait_polls; the array's status word is not visible
 *     to the caller. */
sva_status sva_spec_verify_attn_noalloc(const sva_batch *batch, const void *q, int32_t q_dtype,
                                        int32_t Hq, const sva_paged_kv *kv, float softmax_scale,
                                        void *out, int32_t out_dtype,
                                        const sva_verify_opts *opts, void *stream);

/* Append, then verify, in one call: the same results as sva_kv_append(batch,
 * k_new, v_new, src_dtype, kv) followed by sva_spec_verify_attn (draft_mask
 * NULL) or sva_spec_verify_attn_tree (draft_mask given) on the same stream,
 * cache bytes included ("HeteroReason", workflow Phase 3: the speculated rows
 * enter the cache and are verified in the same pass).  On the split-KV
 * kernels the appended rows are written by the workgroup that streams their
 * page, before it starts streaming, so the step needs one launch fewer; for
 * long speculated steps (the row-block kernel), and where a kv head's query
 * heads are split over workgroups (each of them reads the new rows), the
 * append is its own launch.
 *   k_new, v_new  device [T, Hkv, d] of src_dtype (SVA_F32 or SVA_BF16), as for
 *                 sva_kv_append
 * Every other argument, and every limit, is as for sva_spec_verify_attn (or
 * the tree variant when draft_mask is given). */
sva_status sva_spec_verify_attn_append(const sva_batch *batch, const void *q, int32_t q_dtype,
                                       int32_t Hq, const sva_paged_kv *kv, const void *k_new,
                                       const void *v_new, int32_t src_dtype,
                                       const uint32_t *draft_mask, float softmax_scale,
                                       void *out, int32_t out_dtype,
                                       const sva_verify_opts *opts, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Greedy tree acceptance.  Logit rows as for sva_accept_prefix: sequence b
 * owns k_b + 1 rows from cu_q[b] + b; row 0 scores the token after the
 * committed context, row 1 + i the token after node i.  From the root, the
 * walk moves to the child whose draft token equals the argmax of the current
 * node's row (the lowest index when several children carry it) and stops
 * when none does.
 *   argmax_ids   device [T + B] int32 (written), as for sva_accept_prefix
 *   accept_len   device [B] int32 (written): n_b, nodes on the accepted branch
 *   next_token   device [B] int32 (written): the target's token at the last
 *                accepted node (the root when n_b = 0)
 *   accept_path  device [T] int32 (written): entries cu_q[b] .. cu_q[b]+n_b-1
 *                hold the accepted nodes from the root down, the rest -1
 *   workspace    >= sva_accept_workspace_bytes(batch, V) bytes
 * The step emits the branch's draft tokens, then next_token: n_b + 1 tokens. */
sva_status sva_accept_tree(const sva_batch *batch, const float *logits, int32_t V,
                           const int32_t *draft_ids, const int32_t *parents, int32_t *argmax_ids,
                           int32_t *accept_len, int32_t *next_token, int32_t *accept_path,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Commit of the accepted branch: for every sequence and kv head, the K/V rows
 * (and INT8 scales) at positions S_b + accept_path[cu_q[b] + j] move to
 * S_b + j, j < accept_len[b], so the cache holds one linear sequence again
 * ("HeteroReason", KVMU: rejected speculative history is discarded by a
 * pointer move; the surviving branch is first made contiguous).  Rows are
 * read before any is written, so overlapping moves are safe.  Path entries
 * outside j+1 .. k_b-1 leave row j in place (a chain's path is the
 * identity).  ctx_lens is not changed: the caller commits
 * S_b += n_b.  The pages of positions S_b .. S_b + k_b - 1 must belong to
 * sequence b alone. */
sva_status sva_kv_commit_path(const sva_batch *batch, const int32_t *accept_len,
                              const int32_t *accept_path, const sva_paged_kv *kv, void *stream);

/* Tree acceptance and the commit of the accepted branch in one call: the same
 * results as sva_accept_tree followed by sva_kv_commit_path with its
 * accept_len and accept_path ("Decoding Speculative Decoding from First
 * Principles", section "Tree based verification"; "HeteroReason", KVMU).  The
 * walk of each sequence runs in the workgroups that move its rows, so the
 * branch is committed without a launch of its own.  Arguments as for those
 * two calls (every output written as they write it; workspace >=
 * sva_accept_workspace_bytes(batch, V) bytes, 8-byte aligned); K/V buffers
 * 16-byte aligned, d in {64, 128, 256}.  Errors: SVA_ERR_INVALID_ARG for NULL
 * pointers, a short or misaligned workspace or misaligned K/V buffers;
 * SVA_ERR_UNSUPPORTED for other d or B * Hkv above 2^31 - 1. */
sva_status sva_accept_tree_commit(const sva_batch *batch, const float *logits, int32_t V,
                                  const int32_t *draft_ids, const int32_t *parents,
                                  const sva_paged_kv *kv, int32_t *argmax_ids,
                                  int32_t *accept_len, int32_t *next_token,
                                  int32_t *accept_path, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* ---- Stochastic acceptance -------------------------------------------------
 * "Decoding Speculative Decoding from First Principles", section "How does
 * this drafter maintain the same distribution of the target?": with p the
 * target's and q the drafter's distribution at a draft position and x the
 * drafted token, the draft is accepted with probability min(1, p(x)/q(x));
 * at the first rejection the emitted token is sampled from the residual
 * max(p - q, 0), renormalised, and the pass stops; the emitted tokens are then
 * distributed exactly as the target's.  If every draft is accepted the +1
 * token is sampled from p after the last draft.  p = softmax(target_logits /
 * temperature), q = softmax(draft_logits / temperature).  The random numbers
 * are inputs, so the call is deterministic:
 *   target_logits  device [T + B, V] fp32, rows as for sva_accept_prefix
 *   draft_logits   device [T, V] fp32: the drafter's logits at each draft
 *   draft_ids      device [T] int32: the drafted tokens
 *   u_accept       device [T] fp32 in [0, 1): draft j is accepted iff
 *                  u_accept[j] < p(x)/q(x) (q(x) = 0 accepts, p(x) = 0 rejects)
 *   u_sample       device [B] fp32 in [0, 1): the emitted token is the first
 *                  index whose running sum of weights exceeds u * their total
 *                  (residual weights after a rejection -- p if the residual is
 *                  zero everywhere -- else p of the row after the last draft)
 *   accept_len     device [B] int32 (written): accepted drafts n_b
 *   next_token     device [B] int32 (written): the sampled token
 *   workspace      >= sva_accept_stochastic_workspace_bytes(batch, V) bytes,
 *                  16-byte aligned, no initialisation needed
 * Logits must not be NaN (-inf marks a token of probability zero).  Decisions
 * use fp32 arithmetic: where u lies within rounding of p/q, or u_sample * total
 * within rounding of a running-sum boundary, either neighbouring outcome may
 * be returned. */
size_t sva_accept_stochastic_workspace_bytes(const sva_batch *batch, int32_t V);
sva_status sva_accept_stochastic(const sva_batch *batch, const float *target_logits,
                                 const float *draft_logits, int32_t V, float temperature,
                                 const int32_t *draft_ids, const float *u_accept,
                                 const float *u_sample, int32_t *accept_len, int32_t *next_token,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* ---- KV-cache pointer management --------------------------------------------
 * "HeteroReason", KV Cache Management Unit (Fig. 7): each sequence's cache is
 * tracked by a pointer triplet -- valid (the last verified context boundary),
 * curr (the step under verification) and ahead (the step-ahead speculation
 * frontier) -- moved by the controller's modes.  Rejected speculative history
 * is discarded by moving pointers only.  The Prefix mode is the token-level
 * form used with the accept calls: the first n_b drafts are kept, the rest
 * rolled back.  Keeping the triplets on the device lets a verification loop
 * commit from accept_len without a host round trip. */
typedef enum {
  SVA_KVMU_INIT = 0,       /* valid, curr, ahead <- arg                          */
  SVA_KVMU_SPECULATE = 1,  /* ahead <- ahead + max(arg, 0)                       */
  SVA_KVMU_ACCEPT = 2,     /* valid <- curr, curr <- ahead                       */
  SVA_KVMU_ROLLBACK = 3,   /* curr, ahead <- valid                               */
  SVA_KVMU_PREFIX = 4      /* valid <- min(valid + max(arg, 0), ahead);
                              curr, ahead <- valid                               */
} sva_kvmu_mode;

/* Apply one mode to every sequence's triplet.
 *   mode          device [B] int32 per-sequence modes, or NULL to apply
 *                 uniform_mode to all (an unknown per-sequence mode leaves that
 *                 sequence unchanged)
 *   arg           device [B] int32 (position or count), or NULL for 0
 *   state         device [B, 3] int32 (valid, curr, ahead), updated in place
 *   ctx_lens      device [B] int32 or NULL: receives the new valid pointers
 *                 (the S_b of the next verification step) */
sva_status sva_kvmu_apply(int32_t B, const int32_t *mode, int32_t uniform_mode,
                          const int32_t *arg, int32_t *state, int32_t *ctx_lens, void *stream);

/* Pages of the speculative history.  The management unit discards rejected
 * speculation by moving pointers; these two calls keep the pages in step, on
 * the device, so a whole verification loop (allocate, append and verify,
 * accept, commit, reclaim) runs without a host round trip and can be captured
 * in a HIP graph.  The caller owns the free list and the pages; the library
 * only moves page ids.  Both calls use one workgroup and fixed orders:
 * sequence by sequence, logical page by logical page.
 *   block_table   device [B, max_pages_per_seq] int32 (entries < 0: unassigned)
 *   free_list     device [free_capacity] int32 page ids; entries
 *                 0 .. *free_count - 1 are free pages, the top is the last
 *   free_count    device int32 [1], updated in place
 *
 * Reclaim: for every sequence b, every logical page j with 16 j >= valid_lens[b]
 * (wholly at or past the valid pointer) that holds a page is appended to the
 * list (after its current entries) and its entry set to -1.  Entries past
 * free_capacity are not stored, but *free_count still counts them (a count
 * above the capacity means the list overflowed).
 *   valid_lens    device [B] int32: the committed lengths (for instance the
 *                 ctx_lens that sva_kvmu_apply wrote) */
sva_status sva_kv_reclaim_pages(int32_t B, const int32_t *valid_lens, int32_t *block_table,
                                int32_t max_pages_per_seq, int32_t *free_list,
                                int32_t *free_count, int32_t free_capacity, void *stream);

/* Allocate: before a step appends rows S_b .. S_b + k_b - 1, every unassigned
 * logical page j with 16 j < S_b + k_b takes the page on top of the list
 * (free_list[*free_count - 1] first).  If the list runs out, the remaining
 * entries stay unassigned (the append then skips their rows) and *free_count
 * ends at 0.  *free_count must not exceed free_capacity. */
sva_status sva_kv_alloc_pages(const sva_batch *batch, int32_t *block_table,
                              int32_t max_pages_per_seq, const int32_t *free_list,
                              int32_t *free_count, int32_t free_capacity, void *stream);

/* ---- Measurement ------------------------------------------------------------
 * Streaming-read probe: the rate at which one kernel reads HBM on this device,
 * the achievable ceiling of the verification kernel's KV stream (every KV byte
 * is read once per call; "Decoding Speculative Decoding from First
 * Principles", prerequisite section on the roofline: decode is bound by
 * reading the cache from memory).  Not a step of the method.
 *   buf             device, 16-byte aligned; `bytes` (a multiple of 1024) are
 *                   read once with non-temporal 16-byte loads
 *   mode            0: into registers (8 loads in flight per thread);
 *                   1: through global -> LDS copies, the verification kernel's
 *                   path (up to 32 KB in flight per wave);
 *                   2: as 1 over 4 KB pages in a scattered order, the access
 *                   pattern of a paged cache (`bytes` must be 4096 times a
 *                   power of two; position j reads page j * c mod n for a
 *                   fixed odd c)
 *   num_workgroups  1 .. 65536 workgroups of 256 threads, each reading one
 *                   contiguous range (mode 2: of the page order)
 *   sink            device [num_workgroups * 4] uint32 (written: one word per
 *                   wave, so no load is dead) */
sva_status sva_stream_read_probe(const void *buf, size_t bytes, int32_t mode,
                                 int32_t num_workgroups, uint32_t *sink, void *stream);

const char *sva_status_string(sva_status status);
const char *sva_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
