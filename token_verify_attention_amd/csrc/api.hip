// C ABI of libspecverify: argument validation, device checks and dispatch.
// Every entry point checks what the host can see before enqueuing anything;
// see include/specverify.h for the contract of each call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"
#include "specverify.h"

// Static scratch of sva_spec_verify_attn_noalloc: one array per device, loaded
// with the code object and held until the process ends -- the attention
// workspace (completion counters, status word, partial slots) of callers that
// cannot allocate.  Kernels get its device address, taken once per device with
// hipGetSymbolAddress; in host code the array's name is not a device address.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

sva_status fail(sva_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sva_status fail(sva_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

sva_status hip_fail(hipError_t e, const char* where) {
  return fail(SVA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
struct DeviceInfo {
  bool checked = false;
  bool gfx950 = false;
  int num_cus = 0;
  std::string arch;
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Info of the current device; false (with the error set) if unusable.
sva_status current_device(const DeviceInfo** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SVA_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    d.arch = prop.gcnArchName;
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.num_cus = prop.multiProcessorCount;
    d.checked = true;
  }
  if (!d.gfx950) return fail(SVA_ERR_UNSUPPORTED, "device arch %s is not gfx950", d.arch.c_str());
  *out = &d;
  return SVA_OK;
}

constexpr int kMaxDrafts = 16;          // drafts per sequence, most entry points
constexpr int kMaxDraftsLong = 1024;    // attention and append (long speculated steps)

sva_status check_batch(const sva_batch* b, int max_drafts = kMaxDrafts) {
  if (!b) return fail(SVA_ERR_INVALID_ARG, "batch is NULL");
  if (b->B < 0) return fail(SVA_ERR_INVALID_ARG, "B = %d < 0", b->B);
  if (b->B > 4096) return fail(SVA_ERR_UNSUPPORTED, "B = %d > 4096", b->B);
  if (b->total_q < 0) return fail(SVA_ERR_INVALID_ARG, "total_q = %d < 0", b->total_q);
  if (b->B > 0 && (!b->ctx_lens || !b->cu_q))
    return fail(SVA_ERR_INVALID_ARG, "ctx_lens / cu_q is NULL");
  if (b->total_q > 0 && b->max_q < 1)
    return fail(SVA_ERR_INVALID_ARG, "max_q = %d but total_q = %d", b->max_q, b->total_q);
  if (b->max_q > max_drafts)
    return fail(SVA_ERR_UNSUPPORTED, "max_q = %d > %d", b->max_q, max_drafts);
  if (b->max_q < 0) return fail(SVA_ERR_INVALID_ARG, "max_q = %d < 0", b->max_q);
  if (int64_t(b->B) * b->max_q < b->total_q)
    return fail(SVA_ERR_INVALID_ARG, "total_q = %d exceeds B * max_q", b->total_q);
  if (b->max_len < 0) return fail(SVA_ERR_INVALID_ARG, "max_len = %d < 0", b->max_len);
  return SVA_OK;
}

sva_status check_kv(const sva_paged_kv* kv, bool need_scales) {
  if (!kv) return fail(SVA_ERR_INVALID_ARG, "kv is NULL");
  if (!kv->k || !kv->v || !kv->block_table)
    return fail(SVA_ERR_INVALID_ARG, "kv k / v / block_table is NULL");
  if (kv->page_size != 16) return fail(SVA_ERR_UNSUPPORTED, "page_size = %d != 16", kv->page_size);
  if (kv->Hkv < 1) return fail(SVA_ERR_INVALID_ARG, "Hkv = %d", kv->Hkv);
  if (kv->num_pages < 1) return fail(SVA_ERR_INVALID_ARG, "num_pages = %d", kv->num_pages);
  if (kv->max_pages_per_seq < 1)
    return fail(SVA_ERR_INVALID_ARG, "max_pages_per_seq = %d", kv->max_pages_per_seq);
  if (kv->kv_dtype != SVA_F32 && kv->kv_dtype != SVA_BF16 && kv->kv_dtype != SVA_INT8)
    return fail(SVA_ERR_UNSUPPORTED, "kv_dtype = %d", kv->kv_dtype);
  if (need_scales && kv->kv_dtype == SVA_INT8 && (!kv->k_scale || !kv->v_scale))
    return fail(SVA_ERR_INVALID_ARG, "INT8 cache without k_scale / v_scale");
  return SVA_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---- static scratch of sva_spec_verify_attn_noalloc --------------------------
// Counters and status word at the start of the workspace (must start at zero).
constexpr int kScratchClearWords = (2 * 4096 * 4 + 256) / 4;

__global__ void clear_words_kernel(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

struct ScratchSlot {
  bool ready = false;
  void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address.  The first call on a device looks the
// address up and clears the counters on `stream` (a kernel, so the clear is
// ordered before the call's own launch and may be captured into a graph).
sva_status scratch_for_current_device(void** out, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SVA_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& sl = g_scratch[dev];
  if (!sl.ready) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    hipLaunchKernelGGL(clear_words_kernel, dim3((kScratchClearWords + 255) / 256), dim3(256), 0,
                       stream, static_cast<int32_t*>(ptr), kScratchClearWords);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
    sl.ptr = ptr;
    sl.ready = true;
  }
  *out = sl.ptr;
  return SVA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

namespace sva {
// Tree walk and branch commit in one launch after the argmax (tree.hip).
hipError_t launch_accept_tree_commit(const sva_batch* batch, const float* logits, int V,
                                     const int32_t* draft_ids, const int32_t* parents,
                                     const sva_paged_kv* kv, int32_t* argmax_ids,
                                     int32_t* accept_len, int32_t* next_token,
                                     int32_t* accept_path, const AcceptPlan& plan,
                                     void* workspace, hipStream_t st);
}  // namespace sva

extern "C" {

const char* sva_status_string(sva_status s) {
  switch (s) {
    case SVA_OK: return "SVA_OK";
    case SVA_ERR_INVALID_ARG: return "SVA_ERR_INVALID_ARG";
    case SVA_ERR_UNSUPPORTED: return "SVA_ERR_UNSUPPORTED";
    case SVA_ERR_HIP: return "SVA_ERR_HIP";
  }
  return "unknown sva_status";
}

const char* sva_last_error(void) { return g_last_error.c_str(); }

sva_status sva_kv_quant_int8(const void* x, int32_t src_dtype, int64_t rows, int32_t d,
                             int8_t* codes, uint16_t* scales, void* stream) {
  g_last_error.clear();
  if (rows < 0) return fail(SVA_ERR_INVALID_ARG, "rows = %lld < 0", (long long)rows);
  if (src_dtype != SVA_F32 && src_dtype != SVA_BF16)
    return fail(SVA_ERR_UNSUPPORTED, "src_dtype = %d", src_dtype);
  if (d != 64 && d != 128 && d != 256) return fail(SVA_ERR_UNSUPPORTED, "d = %d", d);
  if (rows == 0) return SVA_OK;
  if (!x || !codes || !scales) return fail(SVA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(x) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 1))
    return fail(SVA_ERR_INVALID_ARG, "x / codes must be 16-byte aligned, scales 2-byte aligned");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_kv_quant_int8(x, src_dtype, rows, d, codes, scales, as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "kv_quant_int8 launch");
}

sva_status sva_kv_append(const sva_batch* batch, const void* k_new, const void* v_new,
                         int32_t src_dtype, const sva_paged_kv* kv, void* stream) {
  g_last_error.clear();
  if (sva_status s = check_batch(batch, kMaxDraftsLong)) return s;
  if (sva_status s = check_kv(kv, true)) return s;
  if (src_dtype != SVA_F32 && src_dtype != SVA_BF16)
    return fail(SVA_ERR_UNSUPPORTED, "src_dtype = %d", src_dtype);
  if (kv->d != 64 && kv->d != 128 && kv->d != 256) return fail(SVA_ERR_UNSUPPORTED, "d = %d", kv->d);
  if (batch->total_q == 0 || batch->B == 0) return SVA_OK;
  if (!k_new || !v_new) return fail(SVA_ERR_INVALID_ARG, "k_new / v_new is NULL");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(kv->k) || !aligned16(kv->v))
    return fail(SVA_ERR_INVALID_ARG, "K/V buffers must be 16-byte aligned");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_kv_append(batch, k_new, v_new, src_dtype, kv, as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "kv_append launch");
}

static sva_status check_attn_shape(const sva_batch* batch, const sva_paged_kv* kv, int32_t Hq,
                                   const sva_verify_opts* opts, bool tree) {
  if (sva_status s = check_batch(batch, tree ? 32 : kMaxDraftsLong)) return s;
  if (sva_status s = check_kv(kv, true)) return s;
  if (kv->d != 64 && kv->d != 128) return fail(SVA_ERR_UNSUPPORTED, "d = %d (64 or 128)", kv->d);
  if (Hq < 1 || Hq % kv->Hkv != 0)
    return fail(SVA_ERR_INVALID_ARG, "Hq = %d is not a multiple of Hkv = %d", Hq, kv->Hkv);
  const int64_t G = Hq / kv->Hkv;
  // more than 16 drafts or 128 query rows per pair: the row-block MFMA kernel only
  const bool valu = kv->kv_dtype == SVA_F32 || (opts && opts->path == 1);
  if (valu && (batch->max_q > kMaxDrafts || G * batch->max_q > 128))
    return fail(SVA_ERR_UNSUPPORTED,
                "max_q = %d, max_q * G = %lld: past 16 drafts or 128 rows only bf16 / INT8 "
                "caches on the MFMA path", batch->max_q, (long long)(G * batch->max_q));
  if (G * batch->max_q > (int64_t(1) << 24))
    return fail(SVA_ERR_UNSUPPORTED, "max_q * G = %lld too large", (long long)(G * batch->max_q));
  const int64_t pages_ub =
      int64_t(batch->B) * kv->Hkv * std::min<int64_t>(kv->max_pages_per_seq, (int64_t(batch->max_len) + 15) / 16);
  // plus the work split's fixed cost per pair (at most 64 pages' worth)
  if (pages_ub + int64_t(batch->B) * kv->Hkv * 64 >= (int64_t(1) << 31) - 1)
    return fail(SVA_ERR_UNSUPPORTED, "B * Hkv * pages = %lld too large", (long long)pages_ub);
  return SVA_OK;
}

size_t sva_verify_workspace_bytes(const sva_batch* batch, const sva_paged_kv* kv, int32_t Hq,
                                  const sva_verify_opts* opts) {
  g_last_error.clear();
  if (check_attn_shape(batch, kv, Hq, opts, false) != SVA_OK) return 0;
  const DeviceInfo* dev;
  if (current_device(&dev) != SVA_OK) return 0;
  return sva::plan_verify_attn(batch, kv, Hq, dev->num_cus, opts).total_bytes;
}

static sva_status verify_attn(const sva_batch* batch, const void* q, int32_t q_dtype, int32_t Hq,
                              const sva_paged_kv* kv, const uint32_t* draft_mask,
                              float softmax_scale, void* out, int32_t out_dtype,
                              const sva_verify_opts* opts, void* workspace,
                              size_t workspace_bytes, void* stream,
                              const void* k_new = nullptr, const void* v_new = nullptr,
                              int32_t src_dtype = SVA_BF16,
                              size_t max_bytes = size_t(1) << 30) {
  if (sva_status s = check_attn_shape(batch, kv, Hq, opts, draft_mask != nullptr)) return s;
  if (q_dtype != SVA_F32 && q_dtype != SVA_BF16)
    return fail(SVA_ERR_UNSUPPORTED, "q_dtype = %d", q_dtype);
  if (out_dtype != SVA_F32 && out_dtype != SVA_BF16)
    return fail(SVA_ERR_UNSUPPORTED, "out_dtype = %d", out_dtype);
  if (!(softmax_scale == softmax_scale) || softmax_scale == 0.f || !std::isfinite(softmax_scale))
    return fail(SVA_ERR_INVALID_ARG, "softmax_scale must be finite and non-zero");
  int path = opts ? opts->path : 0;
  if (path < 0 || path > 2) return fail(SVA_ERR_INVALID_ARG, "opts->path = %d", path);
  if (opts && (opts->num_workgroups < 0 || opts->num_workgroups > 4096))
    return fail(SVA_ERR_INVALID_ARG, "opts->num_workgroups = %d (0 .. 4096)", opts->num_workgroups);
  if (batch->total_q == 0 || batch->B == 0) return SVA_OK;
  if (!q || !out) return fail(SVA_ERR_INVALID_ARG, "q / out is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(kv->k) || !aligned16(kv->v))
    return fail(SVA_ERR_INVALID_ARG, "q / out / K / V must be 16-byte aligned");
  if (kv->kv_dtype == SVA_INT8 && (!aligned16(kv->k_scale) || !aligned16(kv->v_scale)))
    return fail(SVA_ERR_INVALID_ARG, "INT8 scales must be 16-byte aligned");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  const sva::AttnPlan plan = sva::plan_verify_attn(batch, kv, Hq, dev->num_cus, opts, max_bytes);
  if (!workspace || workspace_bytes < plan.total_bytes)
    return fail(SVA_ERR_INVALID_ARG, "workspace of %zu bytes < %zu needed", workspace_bytes,
                plan.total_bytes);
  if (!aligned16(workspace)) return fail(SVA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  hipError_t e = sva::launch_verify_attn(batch, q, q_dtype, Hq, kv, draft_mask, softmax_scale, out,
                                         out_dtype, path, plan, workspace, as_stream(stream),
                                         k_new, v_new, src_dtype);
  return e == hipSuccess ? SVA_OK : hip_fail(e, "spec_verify_attn launch");
}

sva_status sva_spec_verify_attn(const sva_batch* batch, const void* q, int32_t q_dtype,
                                int32_t Hq, const sva_paged_kv* kv, float softmax_scale,
                                void* out, int32_t out_dtype, const sva_verify_opts* opts,
                                void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return verify_attn(batch, q, q_dtype, Hq, kv, nullptr, softmax_scale, out, out_dtype, opts,
                     workspace, workspace_bytes, stream);
}

sva_status sva_spec_verify_attn_noalloc(const sva_batch* batch, const void* q, int32_t q_dtype,
                                        int32_t Hq, const sva_paged_kv* kv, float softmax_scale,
                                        void* out, int32_t out_dtype, const sva_verify_opts* opts,
                                        void* stream) {
  g_last_error.clear();
  if (sva_status s = check_attn_shape(batch, kv, Hq, opts, false)) return s;
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  // the row-block kernel's key slices are limited to the scratch; the split
  // kernel's partials are not (a shape that needs more is refused)
  const size_t need =
      sva::plan_verify_attn(batch, kv, Hq, dev->num_cus, opts, kScratchBytes).total_bytes;
  if (need > kScratchBytes)
    return fail(SVA_ERR_UNSUPPORTED,
                "this call needs %zu bytes of workspace; the static scratch holds %zu "
                "(fewer workgroups or fewer query rows per pair fit)",
                need, kScratchBytes);
  void* ws = nullptr;
  if (sva_status s = scratch_for_current_device(&ws, as_stream(stream))) return s;
  return verify_attn(batch, q, q_dtype, Hq, kv, nullptr, softmax_scale, out, out_dtype, opts, ws,
                     kScratchBytes, stream, nullptr, nullptr, SVA_BF16, kScratchBytes);
}

sva_status sva_spec_verify_attn_append(const sva_batch* batch, const void* q, int32_t q_dtype,
                                       int32_t Hq, const sva_paged_kv* kv, const void* k_new,
                                       const void* v_new, int32_t src_dtype,
                                       const uint32_t* draft_mask, float softmax_scale,
                                       void* out, int32_t out_dtype, const sva_verify_opts* opts,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (sva_status s = check_batch(batch, kMaxDraftsLong)) return s;
  if (sva_status s = check_kv(kv, true)) return s;
  if (src_dtype != SVA_F32 && src_dtype != SVA_BF16)
    return fail(SVA_ERR_UNSUPPORTED, "src_dtype = %d", src_dtype);
  if (batch->total_q > 0 && batch->B > 0) {
    if (!k_new || !v_new) return fail(SVA_ERR_INVALID_ARG, "k_new / v_new is NULL");
    if (!aligned16(k_new) || !aligned16(v_new))
      return fail(SVA_ERR_INVALID_ARG, "k_new / v_new must be 16-byte aligned");
  }
  return verify_attn(batch, q, q_dtype, Hq, kv, draft_mask, softmax_scale, out, out_dtype, opts,
                     workspace, workspace_bytes, stream, k_new, v_new, src_dtype);
}

sva_status sva_spec_verify_attn_tree(const sva_batch* batch, const void* q, int32_t q_dtype,
                                     int32_t Hq, const sva_paged_kv* kv,
                                     const uint32_t* draft_mask, float softmax_scale, void* out,
                                     int32_t out_dtype, const sva_verify_opts* opts,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (batch && batch->total_q > 0 && !draft_mask)
    return fail(SVA_ERR_INVALID_ARG, "draft_mask is NULL");
  return verify_attn(batch, q, q_dtype, Hq, kv, draft_mask, softmax_scale, out, out_dtype, opts,
                     workspace, workspace_bytes, stream);
}

sva_status sva_tree_masks(const sva_batch* batch, const int32_t* parents, uint32_t* masks,
                          void* stream) {
  g_last_error.clear();
  if (sva_status s = check_batch(batch)) return s;
  if (batch->total_q == 0 || batch->B == 0) return SVA_OK;
  if (!parents || !masks) return fail(SVA_ERR_INVALID_ARG, "parents / masks is NULL");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_tree_masks(batch, parents, masks, as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "tree_masks launch");
}

size_t sva_accept_workspace_bytes(const sva_batch* batch, int32_t V) {
  g_last_error.clear();
  if (check_batch(batch) != SVA_OK || V < 1) return 0;
  return sva::plan_accept(batch, V).total_bytes;
}

sva_status sva_accept_prefix(const sva_batch* batch, const float* logits, int32_t V,
                             const int32_t* draft_ids, int32_t* argmax_ids, int32_t* accept_len,
                             int32_t* next_token, void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_last_error.clear();
  if (sva_status s = check_batch(batch)) return s;
  if (V < 1) return fail(SVA_ERR_INVALID_ARG, "V = %d < 1", V);
  if (batch->B == 0) return SVA_OK;
  if (!logits || !argmax_ids || !accept_len || !next_token || (batch->total_q > 0 && !draft_ids))
    return fail(SVA_ERR_INVALID_ARG, "NULL pointer");
  const sva::AcceptPlan plan = sva::plan_accept(batch, V);
  if (!workspace || workspace_bytes < plan.total_bytes)
    return fail(SVA_ERR_INVALID_ARG, "workspace of %zu bytes < %zu needed", workspace_bytes,
                plan.total_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 7) != 0)
    return fail(SVA_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_accept_prefix(batch, logits, V, draft_ids, argmax_ids, accept_len,
                                           next_token, plan, workspace, as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "accept_prefix launch");
}

sva_status sva_accept_tree(const sva_batch* batch, const float* logits, int32_t V,
                           const int32_t* draft_ids, const int32_t* parents, int32_t* argmax_ids,
                           int32_t* accept_len, int32_t* next_token, int32_t* accept_path,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (sva_status s = check_batch(batch)) return s;
  if (V < 1) return fail(SVA_ERR_INVALID_ARG, "V = %d < 1", V);
  if (batch->B == 0) return SVA_OK;
  if (!logits || !argmax_ids || !accept_len || !next_token ||
      (batch->total_q > 0 && (!draft_ids || !parents || !accept_path)))
    return fail(SVA_ERR_INVALID_ARG, "NULL pointer");
  const sva::AcceptPlan plan = sva::plan_accept(batch, V);
  if (!workspace || workspace_bytes < plan.total_bytes)
    return fail(SVA_ERR_INVALID_ARG, "workspace of %zu bytes < %zu needed", workspace_bytes,
                plan.total_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 7) != 0)
    return fail(SVA_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_accept_tree(batch, logits, V, draft_ids, parents, argmax_ids,
                                         accept_len, next_token, accept_path, plan, workspace,
                                         as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "accept_tree launch");
}

sva_status sva_accept_tree_commit(const sva_batch* batch, const float* logits, int32_t V,
                                  const int32_t* draft_ids, const int32_t* parents,
                                  const sva_paged_kv* kv, int32_t* argmax_ids,
                                  int32_t* accept_len, int32_t* next_token, int32_t* accept_path,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (sva_status s = check_batch(batch)) return s;
  if (sva_status s = check_kv(kv, true)) return s;
  if (kv->d != 64 && kv->d != 128 && kv->d != 256) return fail(SVA_ERR_UNSUPPORTED, "d = %d", kv->d);
  if (V < 1) return fail(SVA_ERR_INVALID_ARG, "V = %d < 1", V);
  if (batch->B == 0) return SVA_OK;
  if (!logits || !argmax_ids || !accept_len || !next_token ||
      (batch->total_q > 0 && (!draft_ids || !parents || !accept_path)))
    return fail(SVA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(kv->k) || !aligned16(kv->v))
    return fail(SVA_ERR_INVALID_ARG, "K/V buffers must be 16-byte aligned");
  if (int64_t(batch->B) * kv->Hkv > 0x7fffffff)
    return fail(SVA_ERR_UNSUPPORTED, "B * Hkv too large");
  const sva::AcceptPlan plan = sva::plan_accept(batch, V);
  if (!workspace || workspace_bytes < plan.total_bytes)
    return fail(SVA_ERR_INVALID_ARG, "workspace of %zu bytes < %zu needed", workspace_bytes,
                plan.total_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 7) != 0)
    return fail(SVA_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_accept_tree_commit(batch, logits, V, draft_ids, parents, kv,
                                                argmax_ids, accept_len, next_token, accept_path,
                                                plan, workspace, as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "accept_tree_commit launch");
}

size_t sva_accept_stochastic_workspace_bytes(const sva_batch* batch, int32_t V) {
  g_last_error.clear();
  if (check_batch(batch) != SVA_OK || V < 1) return 0;
  return sva::plan_sample(batch, V).total_bytes;
}

sva_status sva_accept_stochastic(const sva_batch* batch, const float* target_logits,
                                 const float* draft_logits, int32_t V, float temperature,
                                 const int32_t* draft_ids, const float* u_accept,
                                 const float* u_sample, int32_t* accept_len, int32_t* next_token,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (sva_status s = check_batch(batch)) return s;
  if (V < 1) return fail(SVA_ERR_INVALID_ARG, "V = %d < 1", V);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(SVA_ERR_INVALID_ARG, "temperature must be finite and > 0");
  if (batch->B == 0) return SVA_OK;
  if (!target_logits || !u_sample || !accept_len || !next_token ||
      (batch->total_q > 0 && (!draft_logits || !draft_ids || !u_accept)))
    return fail(SVA_ERR_INVALID_ARG, "NULL pointer");
  const sva::SamplePlan plan = sva::plan_sample(batch, V);
  if (!workspace || workspace_bytes < plan.total_bytes)
    return fail(SVA_ERR_INVALID_ARG, "workspace of %zu bytes < %zu needed", workspace_bytes,
                plan.total_bytes);
  if (!aligned16(workspace)) return fail(SVA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_accept_stochastic(batch, target_logits, draft_logits, V, temperature,
                                               draft_ids, u_accept, u_sample, accept_len,
                                               next_token, plan, workspace, as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "accept_stochastic launch");
}

sva_status sva_kvmu_apply(int32_t B, const int32_t* mode, int32_t uniform_mode,
                          const int32_t* arg, int32_t* state, int32_t* ctx_lens, void* stream) {
  g_last_error.clear();
  if (B < 0) return fail(SVA_ERR_INVALID_ARG, "B = %d < 0", B);
  if (!mode && (uniform_mode < SVA_KVMU_INIT || uniform_mode > SVA_KVMU_PREFIX))
    return fail(SVA_ERR_INVALID_ARG, "uniform_mode = %d", uniform_mode);
  if (B == 0) return SVA_OK;
  if (!state) return fail(SVA_ERR_INVALID_ARG, "state is NULL");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_kvmu(B, mode, uniform_mode, arg, state, ctx_lens, as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "kvmu_apply launch");
}

sva_status sva_kv_reclaim_pages(int32_t B, const int32_t* valid_lens, int32_t* block_table,
                                int32_t max_pages_per_seq, int32_t* free_list,
                                int32_t* free_count, int32_t free_capacity, void* stream) {
  g_last_error.clear();
  if (B < 0 || B > 4096) return fail(SVA_ERR_INVALID_ARG, "B = %d (0 .. 4096)", B);
  if (max_pages_per_seq < 1)
    return fail(SVA_ERR_INVALID_ARG, "max_pages_per_seq = %d", max_pages_per_seq);
  if (free_capacity < 0) return fail(SVA_ERR_INVALID_ARG, "free_capacity = %d", free_capacity);
  if (B == 0) return SVA_OK;
  if (!valid_lens || !block_table || !free_list || !free_count)
    return fail(SVA_ERR_INVALID_ARG, "NULL pointer");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_kv_reclaim_pages(B, valid_lens, block_table, max_pages_per_seq,
                                              free_list, free_count, free_capacity,
                                              as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "kv_reclaim_pages launch");
}

sva_status sva_kv_alloc_pages(const sva_batch* batch, int32_t* block_table,
                              int32_t max_pages_per_seq, const int32_t* free_list,
                              int32_t* free_count, int32_t free_capacity, void* stream) {
  g_last_error.clear();
  if (sva_status s = check_batch(batch, kMaxDraftsLong)) return s;
  if (max_pages_per_seq < 1)
    return fail(SVA_ERR_INVALID_ARG, "max_pages_per_seq = %d", max_pages_per_seq);
  if (free_capacity < 0) return fail(SVA_ERR_INVALID_ARG, "free_capacity = %d", free_capacity);
  if (batch->B == 0) return SVA_OK;
  if (!block_table || !free_list || !free_count) return fail(SVA_ERR_INVALID_ARG, "NULL pointer");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_kv_alloc_pages(batch, block_table, max_pages_per_seq, free_list,
                                            free_count, free_capacity, as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "kv_alloc_pages launch");
}

sva_status sva_stream_read_probe(const void* buf, size_t bytes, int32_t mode,
                                 int32_t num_workgroups, uint32_t* sink, void* stream) {
  g_last_error.clear();
  if (mode < 0 || mode > 2) return fail(SVA_ERR_INVALID_ARG, "mode = %d (0, 1 or 2)", mode);
  if (mode == 2 && (bytes % 4096 != 0 || ((bytes / 4096) & (bytes / 4096 - 1)) != 0))
    return fail(SVA_ERR_INVALID_ARG, "mode 2: bytes = %zu is not 4096 times a power of two",
                bytes);
  if (num_workgroups < 1 || num_workgroups > 65536)
    return fail(SVA_ERR_INVALID_ARG, "num_workgroups = %d (1 .. 65536)", num_workgroups);
  if (bytes % 1024 != 0) return fail(SVA_ERR_INVALID_ARG, "bytes = %zu is not a multiple of 1024", bytes);
  if (bytes == 0) return SVA_OK;
  if (!buf || !sink) return fail(SVA_ERR_INVALID_ARG, "buf / sink is NULL");
  if (!aligned16(buf)) return fail(SVA_ERR_INVALID_ARG, "buf must be 16-byte aligned");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_stream_read_probe(buf, bytes, mode, num_workgroups, sink,
                                               as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "stream_read_probe launch");
}

sva_status sva_kv_commit_path(const sva_batch* batch, const int32_t* accept_len,
                              const int32_t* accept_path, const sva_paged_kv* kv, void* stream) {
  g_last_error.clear();
  if (sva_status s = check_batch(batch)) return s;
  if (sva_status s = check_kv(kv, true)) return s;
  if (kv->d != 64 && kv->d != 128 && kv->d != 256) return fail(SVA_ERR_UNSUPPORTED, "d = %d", kv->d);
  if (batch->total_q == 0 || batch->B == 0) return SVA_OK;
  if (!accept_len || !accept_path) return fail(SVA_ERR_INVALID_ARG, "accept_len / accept_path is NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v))
    return fail(SVA_ERR_INVALID_ARG, "K/V buffers must be 16-byte aligned");
  if (int64_t(batch->B) * kv->Hkv > 0x7fffffff)
    return fail(SVA_ERR_UNSUPPORTED, "B * Hkv too large");
  const DeviceInfo* dev;
  if (sva_status s = current_device(&dev)) return s;
  hipError_t e = sva::launch_kv_commit_path(batch, accept_len, accept_path, kv, as_stream(stream));
  return e == hipSuccess ? SVA_OK : hip_fail(e, "kv_commit_path launch");
}

}  // extern "C"
