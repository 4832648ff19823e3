// Token-tree verification for gfx950: ancestor masks, greedy tree acceptance
// and the commit of the accepted branch.
//
// "Decoding Speculative Decoding from First Principles", section "Tree based
// verification": the drafter proposes a tree of continuations; tree attention
// relates each draft only to its own lineage; the accepted continuation is the
// longest branch the target agrees with.  A tree of k_b <= 16 nodes is a
// parent array in topological order (parent -1: child of the last committed
// token; otherwise an earlier node); node i's K/V row sits at position S_b + i.
//
//  * tree_masks_kernel: one wave per sequence; lane i holds node i and, after
//    as many rounds as the tree is deep, the bitmask of its lineage (each
//    round ORs in the parent's mask through a cross-lane read).
//  * accept_tree_scan_kernel: one wave per sequence after the chunked argmax
//    of every logit row (shared with prefix acceptance).  Starting at the
//    root, a ballot over the nodes finds the children of the current node
//    whose draft token equals the target's token at that node (row 1 + node;
//    row 0 for the root); the lowest such index is taken.
//  * kv_commit_path_kernel: one workgroup per (sequence, kv head) moves the
//    accepted branch's rows to positions S_b .. S_b + n_b - 1 (HeteroReason's
//    KVMU discards rejected speculative history by moving a pointer; the
//    surviving branch is first made contiguous).  Source and destination rows
//    can overlap (path node j may sit where row j' < j goes), so every source
//    row is staged in LDS before any row is written.
#include "common.h"
#include "launch.h"
#include "accept_keys.h"

namespace sva {

constexpr int kMaxTree = 16;                // nodes per sequence (max_q)
constexpr int kCommitThreads = 256;
constexpr int kMaxRowBytes = 1024;          // d <= 256 values of up to 4 bytes

// Node range [q0, q0 + k) of sequence b, with device values clamped into the
// buffers.
__device__ __forceinline__ void tree_range(const int32_t* cu_q, int T, int max_q, int b, int& q0,
                                           int& k) {
  int a = cu_q[b], e = cu_q[b + 1];
  a = min(max(a, 0), T);
  e = min(max(e, a), T);
  q0 = a;
  k = min(min(e - a, max_q), kMaxTree);
}

// Parent of node i, read as a root when it is not an earlier node.
__device__ __forceinline__ int tree_parent(const int32_t* parents, int q0, int i) {
  const int p = parents[q0 + i];
  return (p >= 0 && p < i) ? p : -1;
}

__global__ __launch_bounds__(kWave) void tree_masks_kernel(const int32_t* __restrict__ cu_q,
                                                           int T, int max_q,
                                                           const int32_t* __restrict__ parents,
                                                           uint32_t* __restrict__ masks) {
  const int b = blockIdx.x;
  const int lane = lane_id();
  int q0, k;
  tree_range(cu_q, T, max_q, b, q0, k);
  const int par = lane < k ? tree_parent(parents, q0, lane) : -1;
  const uint32_t self = lane < k ? (1u << lane) : 0u;
  uint32_t m = self;
  for (int round = 1; round < k; ++round) {   // depth <= k
    const uint32_t pm = uint32_t(__shfl(int(m), par < 0 ? lane : par, kWave));
    m = self | (par >= 0 ? pm : 0u);
  }
  if (lane < k) masks[q0 + lane] = m;
}

// Outputs of the tree walk (nullptr: not written).
struct TreeOut {
  int32_t* argmax_ids;
  int32_t* accept_len;
  int32_t* next_token;
  int32_t* accept_path;
};

// The greedy walk down sequence b's tree, run by one wave: row 0 scores the
// root, row 1 + i the token after node i.  Lane j returns path node j (-1 past
// the accepted branch); n is the branch length.  Writes the outputs unless
// they are nullptr.
__device__ __forceinline__ int tree_walk(const uint64_t* keys, int chunks, int b, int q0, int k,
                                         const int32_t* draft_ids, const int32_t* parents,
                                         const TreeOut& o, int& n) {
  const int lane = lane_id();
  const int row0 = q0 + b;
  const int tok = row_tokens_from_keys(keys, chunks, row0, k + 1);
  if (o.argmax_ids && lane <= k) o.argmax_ids[row0 + lane] = tok;
  const int par = lane < k ? tree_parent(parents, q0, lane) : -2;
  const int draft = lane < k ? draft_ids[q0 + lane] : 0;
  int cur = -1, mine = -1;                  // lane j keeps path node j
  n = 0;
  for (int step = 0; step < k; ++step) {
    const int t = __shfl(tok, cur + 1, kWave);
    const uint64_t hit = __ballot(par == cur && draft == t);
    if (!hit) break;
    const int c = __builtin_ctzll(hit);
    if (lane == n) mine = c;
    ++n;
    cur = c;
  }
  const int nxt = __shfl(tok, cur + 1, kWave);
  const int node = lane < n ? mine : -1;
  if (o.accept_path && lane < k) o.accept_path[q0 + lane] = node;
  if (lane == 0) {
    if (o.accept_len) o.accept_len[b] = n;
    if (o.next_token) o.next_token[b] = nxt;
  }
  return node;
}

__global__ __launch_bounds__(kWave) void accept_tree_scan_kernel(
    const uint64_t* __restrict__ keys, int chunks, const int32_t* __restrict__ cu_q, int T,
    int max_q, const int32_t* __restrict__ draft_ids, const int32_t* __restrict__ parents,
    TreeOut o) {
  const int b = blockIdx.x;
  int q0, k, n;
  tree_range(cu_q, T, max_q, b, q0, k);
  tree_walk(keys, chunks, b, q0, k, draft_ids, parents, o, n);
}

struct CommitParams {
  char* k;
  char* v;
  uint16_t* k_scale;
  uint16_t* v_scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* cu_q;
  const int32_t* accept_len;
  const int32_t* accept_path;
  int T, max_q, Hkv, num_pages, max_pages;
  int row_bytes;                            // d * element size, a multiple of 16
};

// Byte offset of position pos of sequence b, kv head g, in a K or V pool.
__device__ __forceinline__ int64_t row_offset(const CommitParams& p, int b, int g, int pos) {
  const int pg = min(max(pos / kPage, 0), p.max_pages - 1);
  const int pid = min(max(p.block_table[int64_t(b) * p.max_pages + pg], 0), p.num_pages - 1);
  return ((int64_t(pid) * p.Hkv + g) * kPage + pos % kPage) * p.row_bytes;
}
__device__ __forceinline__ int64_t scale_index(const CommitParams& p, int b, int g, int pos) {
  return row_offset(p, b, g, pos) / p.row_bytes;
}

// LDS staging of one (sequence, kv head)'s moved rows.
struct CommitLds {
  char k[kMaxTree * kMaxRowBytes];
  char v[kMaxTree * kMaxRowBytes];
  uint16_t sc[2][kMaxTree];
  int src[kMaxTree];                        // the node whose row goes to position S + j
  int n;
};

// Moves the accepted branch of (b, g) once c.src[0 .. n-1] and c.n are set
// (and a barrier has passed): every moved row into LDS, then every row to its
// place.
__device__ __forceinline__ void commit_branch(const CommitParams& p, int b, int g, CommitLds& c) {
  const int tid = threadIdx.x;
  const int S = max(p.ctx_lens[b], 0);
  const int n = c.n;
  const int cpr = p.row_bytes / 16;
  // phase 1: every moved row into LDS
  for (int idx = tid; idx < n * cpr; idx += kCommitThreads) {
    const int j = idx / cpr, ch = idx % cpr;
    if (c.src[j] == j) continue;
    const int64_t off = row_offset(p, b, g, S + c.src[j]) + ch * 16;
    *reinterpret_cast<u32x4*>(c.k + j * p.row_bytes + ch * 16) = *reinterpret_cast<const u32x4*>(p.k + off);
    *reinterpret_cast<u32x4*>(c.v + j * p.row_bytes + ch * 16) = *reinterpret_cast<const u32x4*>(p.v + off);
  }
  if (p.k_scale && tid < n && c.src[tid] != tid) {
    const int64_t si = scale_index(p, b, g, S + c.src[tid]);
    c.sc[0][tid] = p.k_scale[si];
    c.sc[1][tid] = p.v_scale[si];
  }
  __syncthreads();
  // phase 2: rows to positions S .. S + n - 1
  for (int idx = tid; idx < n * cpr; idx += kCommitThreads) {
    const int j = idx / cpr, ch = idx % cpr;
    if (c.src[j] == j) continue;
    const int64_t off = row_offset(p, b, g, S + j) + ch * 16;
    *reinterpret_cast<u32x4*>(p.k + off) = *reinterpret_cast<const u32x4*>(c.k + j * p.row_bytes + ch * 16);
    *reinterpret_cast<u32x4*>(p.v + off) = *reinterpret_cast<const u32x4*>(c.v + j * p.row_bytes + ch * 16);
  }
  if (p.k_scale && tid < n && c.src[tid] != tid) {
    const int64_t si = scale_index(p, b, g, S + tid);
    p.k_scale[si] = c.sc[0][tid];
    p.v_scale[si] = c.sc[1][tid];
  }
}

// Where row j of the committed branch comes from: path node pj when it is a
// later node (a path node never precedes its index), else row j itself.
__device__ __forceinline__ int branch_source(int j, int n, int k, int pj) {
  return (j < n && pj > j && pj < k) ? pj : j;
}

__global__ __launch_bounds__(kCommitThreads) void kv_commit_path_kernel(CommitParams p) {
  __shared__ __attribute__((aligned(16))) CommitLds c;
  const int b = blockIdx.x / p.Hkv;
  const int g = blockIdx.x % p.Hkv;
  const int tid = threadIdx.x;
  int q0, k;
  tree_range(p.cu_q, p.T, p.max_q, b, q0, k);
  const int n = min(max(p.accept_len[b], 0), k);
  if (tid < kMaxTree) c.src[tid] = branch_source(tid, n, k, tid < n ? p.accept_path[q0 + tid] : -1);
  if (tid == 0) c.n = n;
  __syncthreads();
  commit_branch(p, b, g, c);
}

// Tree walk and branch commit in one launch: one workgroup per (sequence, kv
// head); its first wave walks the tree (the kv-head-0 workgroup writes the
// acceptance outputs), the workgroup then moves that head's branch rows.  The
// same operations as accept_tree_scan_kernel followed by kv_commit_path_kernel.
__global__ __launch_bounds__(kCommitThreads) void accept_tree_commit_kernel(
    const uint64_t* __restrict__ keys, int chunks, const int32_t* __restrict__ draft_ids,
    const int32_t* __restrict__ parents, TreeOut o, CommitParams p) {
  __shared__ __attribute__((aligned(16))) CommitLds c;
  const int b = blockIdx.x / p.Hkv;
  const int g = blockIdx.x % p.Hkv;
  const int tid = threadIdx.x;
  int q0, k;
  tree_range(p.cu_q, p.T, p.max_q, b, q0, k);
  if (tid < kWave) {
    const TreeOut none{nullptr, nullptr, nullptr, nullptr};
    int n;
    const int node = tree_walk(keys, chunks, b, q0, k, draft_ids, parents, g == 0 ? o : none, n);
    if (tid < kMaxTree) c.src[tid] = branch_source(tid, n, k, node);
    if (tid == 0) c.n = n;
  }
  __syncthreads();
  commit_branch(p, b, g, c);
}

hipError_t launch_tree_masks(const sva_batch* batch, const int32_t* parents, uint32_t* masks,
                             hipStream_t st) {
  hipLaunchKernelGGL(tree_masks_kernel, dim3(batch->B), dim3(kWave), 0, st, batch->cu_q,
                     batch->total_q, batch->max_q, parents, masks);
  return hipGetLastError();
}

hipError_t launch_accept_tree(const sva_batch* batch, const float* logits, int V,
                              const int32_t* draft_ids, const int32_t* parents,
                              int32_t* argmax_ids, int32_t* accept_len, int32_t* next_token,
                              int32_t* accept_path, const AcceptPlan& plan, void* workspace,
                              hipStream_t st) {
  uint64_t* keys = static_cast<uint64_t*>(workspace);
  hipError_t e = launch_argmax_keys(logits, V, plan, keys, st);
  if (e != hipSuccess) return e;
  const TreeOut o{argmax_ids, accept_len, next_token, accept_path};
  hipLaunchKernelGGL(accept_tree_scan_kernel, dim3(batch->B), dim3(kWave), 0, st, keys,
                     plan.chunks, batch->cu_q, batch->total_q, batch->max_q, draft_ids, parents,
                     o);
  return hipGetLastError();
}

static CommitParams commit_params(const sva_batch* batch, const int32_t* accept_len,
                                  const int32_t* accept_path, const sva_paged_kv* kv) {
  CommitParams p;
  p.k = static_cast<char*>(kv->k);
  p.v = static_cast<char*>(kv->v);
  const bool i8 = kv->kv_dtype == SVA_INT8;
  p.k_scale = i8 ? static_cast<uint16_t*>(kv->k_scale) : nullptr;
  p.v_scale = i8 ? static_cast<uint16_t*>(kv->v_scale) : nullptr;
  p.block_table = kv->block_table;
  p.ctx_lens = batch->ctx_lens;
  p.cu_q = batch->cu_q;
  p.accept_len = accept_len;
  p.accept_path = accept_path;
  p.T = batch->total_q;
  p.max_q = batch->max_q;
  p.Hkv = kv->Hkv;
  p.num_pages = kv->num_pages;
  p.max_pages = kv->max_pages_per_seq;
  const int es = kv->kv_dtype == SVA_F32 ? 4 : (kv->kv_dtype == SVA_BF16 ? 2 : 1);
  p.row_bytes = kv->d * es;
  return p;
}

hipError_t launch_kv_commit_path(const sva_batch* batch, const int32_t* accept_len,
                                 const int32_t* accept_path, const sva_paged_kv* kv,
                                 hipStream_t st) {
  const CommitParams p = commit_params(batch, accept_len, accept_path, kv);
  hipLaunchKernelGGL(kv_commit_path_kernel, dim3(unsigned(batch->B) * kv->Hkv),
                     dim3(kCommitThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_accept_tree_commit(const sva_batch* batch, const float* logits, int V,
                                     const int32_t* draft_ids, const int32_t* parents,
                                     const sva_paged_kv* kv, int32_t* argmax_ids,
                                     int32_t* accept_len, int32_t* next_token,
                                     int32_t* accept_path, const AcceptPlan& plan,
                                     void* workspace, hipStream_t st) {
  uint64_t* keys = static_cast<uint64_t*>(workspace);
  hipError_t e = launch_argmax_keys(logits, V, plan, keys, st);
  if (e != hipSuccess) return e;
  const TreeOut o{argmax_ids, accept_len, next_token, accept_path};
  const CommitParams p = commit_params(batch, nullptr, nullptr, kv);
  hipLaunchKernelGGL(accept_tree_commit_kernel, dim3(unsigned(batch->B) * kv->Hkv),
                     dim3(kCommitThreads), 0, st, keys, plan.chunks, draft_ids, parents, o, p);
  return hipGetLastError();
}

}  // namespace sva
