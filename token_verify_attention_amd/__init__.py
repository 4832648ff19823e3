"""Python binding of libspecverify, the gfx950 hot path of speculative-decoding
verification.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/specverify.h.  torch supplies
device memory and streams.  If the built library is missing, ``load()`` raises;
nothing here falls back to another implementation.

    import token_verify_attention_amd as tva
    batch = tva.Batch(ctx_lens, cu_q, max_len=...)        # device int32 tensors
    kv = tva.PagedKV(k_pool, v_pool, block_table)          # [P, Hkv, 16, d]
    tva.kv_append(batch, k_new, v_new, kv)
    out = tva.spec_verify_attn(batch, q, kv)
    ids, n, nxt = tva.accept_prefix(batch, logits, draft_ids)
"""
import contextlib
import ctypes
import functools
import inspect
import math
import os

import torch

__all__ = [
    "load", "SvaError", "Batch", "PagedKV", "kv_quant_int8", "kv_append", "spec_verify_attn",
    "verify_workspace_bytes", "accept_prefix", "accept_workspace_bytes", "LIB_PATH",
    "tree_masks", "accept_tree", "kv_commit_path", "accept_tree_commit", "accept_stochastic",
    "accept_stochastic_workspace_bytes", "kvmu_apply", "KVMU_INIT", "KVMU_SPECULATE",
    "KVMU_ACCEPT", "KVMU_ROLLBACK", "KVMU_PREFIX", "verify_status", "STATUS_OFFSET",
    "spec_verify_attn_append", "spec_verify_attn_noalloc", "stream_read_probe",
    "kv_reclaim_pages", "kv_alloc_pages",
]

KVMU_INIT, KVMU_SPECULATE, KVMU_ACCEPT, KVMU_ROLLBACK, KVMU_PREFIX = 0, 1, 2, 3, 4

# The built library; TVA_LIB names another build of it (a sanitizer build in
# the CPU tests).  Nothing falls back when the file is missing.
LIB_PATH = os.environ.get("TVA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                    "_lib", "libspecverify.so")

SVA_F32, SVA_BF16, SVA_F16, SVA_INT8 = 0, 1, 2, 3
SVA_OK, SVA_ERR_INVALID_ARG, SVA_ERR_UNSUPPORTED, SVA_ERR_HIP = 0, 1, 2, 3
_DTYPE = {torch.float32: SVA_F32, torch.bfloat16: SVA_BF16, torch.float16: SVA_F16,
          torch.int8: SVA_INT8}

PATH_AUTO, PATH_VALU, PATH_MFMA = 0, 1, 2


class SvaError(RuntimeError):
    def __init__(self, func, status, detail):
        self.status = status
        super().__init__(f"{func}: {_status_name(status)}: {detail}")


class _PagedKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


class _Batch(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("ctx_lens", ctypes.c_void_p), ("cu_q", ctypes.c_void_p),
                ("total_q", ctypes.c_int32), ("max_q", ctypes.c_int32),
                ("max_len", ctypes.c_int32)]


class _Opts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("num_workgroups", ctypes.c_int32),
                ("wait_polls", ctypes.c_int32)]


# Byte offset of the attention workspace's status word (after the 2 x 4096
# completion counters); bit 0: a split pair's wait gave up and its rows were
# written as NaN.
STATUS_OFFSET = 2 * 4096 * 4

# With TVA_DEBUG set (non-empty, not "0"), every attention call through this
# binding synchronises its stream and raises if the call set the status word.
DEBUG = os.environ.get("TVA_DEBUG", "") not in ("", "0")


_lib = None


def load():
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m token_verify_attention_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)      # torch is imported first: one HIP runtime
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.sva_status_string.restype = ctypes.c_char_p
        lib.sva_status_string.argtypes = [ctypes.c_int]
        lib.sva_last_error.restype = ctypes.c_char_p
        lib.sva_last_error.argtypes = []
        lib.sva_kv_quant_int8.restype = ctypes.c_int
        lib.sva_kv_quant_int8.argtypes = [vp, i32, i64, i32, vp, vp, vp]
        lib.sva_kv_append.restype = ctypes.c_int
        lib.sva_kv_append.argtypes = [vp, vp, vp, i32, vp, vp]
        lib.sva_verify_workspace_bytes.restype = sz
        lib.sva_verify_workspace_bytes.argtypes = [vp, vp, i32, vp]
        lib.sva_spec_verify_attn.restype = ctypes.c_int
        lib.sva_spec_verify_attn.argtypes = [vp, vp, i32, i32, vp, ctypes.c_float, vp, i32, vp,
                                             vp, sz, vp]
        lib.sva_spec_verify_attn_noalloc.restype = ctypes.c_int
        lib.sva_spec_verify_attn_noalloc.argtypes = [vp, vp, i32, i32, vp, ctypes.c_float, vp,
                                                     i32, vp, vp]
        lib.sva_kv_reclaim_pages.restype = ctypes.c_int
        lib.sva_kv_reclaim_pages.argtypes = [i32, vp, vp, i32, vp, vp, i32, vp]
        lib.sva_kv_alloc_pages.restype = ctypes.c_int
        lib.sva_kv_alloc_pages.argtypes = [vp, vp, i32, vp, vp, i32, vp]
        lib.sva_stream_read_probe.restype = ctypes.c_int
        lib.sva_stream_read_probe.argtypes = [vp, sz, i32, i32, vp, vp]
        lib.sva_accept_workspace_bytes.restype = sz
        lib.sva_accept_workspace_bytes.argtypes = [vp, i32]
        lib.sva_accept_prefix.restype = ctypes.c_int
        lib.sva_accept_prefix.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
        lib.sva_tree_masks.restype = ctypes.c_int
        lib.sva_tree_masks.argtypes = [vp, vp, vp, vp]
        lib.sva_spec_verify_attn_tree.restype = ctypes.c_int
        lib.sva_spec_verify_attn_tree.argtypes = [vp, vp, i32, i32, vp, vp, ctypes.c_float, vp,
                                                  i32, vp, vp, sz, vp]
        lib.sva_spec_verify_attn_append.restype = ctypes.c_int
        lib.sva_spec_verify_attn_append.argtypes = [vp, vp, i32, i32, vp, vp, vp, i32, vp,
                                                    ctypes.c_float, vp, i32, vp, vp, sz, vp]
        lib.sva_accept_tree.restype = ctypes.c_int
        lib.sva_accept_tree.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.sva_kv_commit_path.restype = ctypes.c_int
        lib.sva_kv_commit_path.argtypes = [vp, vp, vp, vp, vp]
        lib.sva_accept_tree_commit.restype = ctypes.c_int
        lib.sva_accept_tree_commit.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                               vp]
        lib.sva_kvmu_apply.restype = ctypes.c_int
        lib.sva_kvmu_apply.argtypes = [i32, vp, i32, vp, vp, vp, vp]
        lib.sva_accept_stochastic_workspace_bytes.restype = sz
        lib.sva_accept_stochastic_workspace_bytes.argtypes = [vp, i32]
        lib.sva_accept_stochastic.restype = ctypes.c_int
        lib.sva_accept_stochastic.argtypes = [vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp,
                                              vp, sz, vp]
        _lib = lib
    return _lib


def _status_name(status):
    return load().sva_status_string(status).decode()


def _check(func, status):
    if status != 0:
        raise SvaError(func, status, load().sva_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Run a call's own allocations (outputs, workspaces) on the stream its
    kernels go to, so the caching allocator never hands their memory to other
    work while those kernels may still run, and a zero fill is ordered before
    them."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapped(*args, **kwargs):
        stream = sig.bind(*args, **kwargs).arguments.get("stream")
        ctx = contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)
        with ctx:
            return fn(*args, **kwargs)
    return wrapped


def verify_status(workspace, stream=None, clear=True):
    """The status word of an attention workspace (synchronises the stream):
    bit 0 is set when a split pair's wait gave up (its rows were written as
    NaN).  clear=True zeroes it afterwards."""
    s = torch.cuda.current_stream(workspace.device) if stream is None else stream
    s.synchronize()
    word = workspace[STATUS_OFFSET:STATUS_OFFSET + 4]
    value = int(word.cpu().view(torch.int32)[0])
    if clear and value:
        with torch.cuda.stream(s):
            word.zero_()
        s.synchronize()
    return value


def _debug_check(name, workspace, stream):
    if DEBUG and workspace is not None:
        v = verify_status(workspace, stream)
        if v:
            raise SvaError(name, 3, f"status word {v:#x}: a split pair's wait gave up; its "
                           "rows are NaN")


def _dtype_code(t, what):
    if t.dtype not in _DTYPE:
        raise TypeError(f"{what}: unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


def _need(t, what, dims=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{what} must have {dims} dimensions, has {t.dim()}")


class Batch:
    """B sequences: ctx_lens [B] (committed rows, excluding the drafts) and
    cu_q [B+1] (prefix sums of the per-sequence draft counts k_b), both device
    int32.  Host bounds: total_q = cu_q[B], max_q >= every k_b, max_len >=
    every S_b + k_b; computed from the tensors when not given (one sync)."""

    def __init__(self, ctx_lens, cu_q, total_q=None, max_q=None, max_len=None):
        _need(ctx_lens, "ctx_lens", 1)
        _need(cu_q, "cu_q", 1)
        if ctx_lens.dtype != torch.int32 or cu_q.dtype != torch.int32:
            raise TypeError("ctx_lens and cu_q must be int32")
        if cu_q.numel() != ctx_lens.numel() + 1:
            raise ValueError("cu_q must have B+1 entries")
        self.ctx_lens, self.cu_q = ctx_lens, cu_q
        self.B = ctx_lens.numel()
        if total_q is None or max_q is None or max_len is None:
            k = (cu_q[1:] - cu_q[:-1]).cpu()
            c = ctx_lens.cpu()
            total_q = int(cu_q[-1].item()) if total_q is None else total_q
            max_q = int(k.max().item()) if (max_q is None and self.B) else (max_q or 0)
            max_len = int((c + k).max().item()) if (max_len is None and self.B) else (max_len or 0)
        self.total_q, self.max_q, self.max_len = int(total_q), int(max_q), int(max_len)

    def _c(self):
        return _Batch(self.B, self.ctx_lens.data_ptr(), self.cu_q.data_ptr(), self.total_q,
                      self.max_q, self.max_len)


class PagedKV:
    """Paged KV cache of one layer: k, v [num_pages, Hkv, 16, d] (float32,
    bfloat16 or int8 codes), k_scale, v_scale [num_pages, Hkv, 16] float16 for
    int8 caches, block_table [B, max_pages_per_seq] int32 (-1 = unused)."""

    def __init__(self, k, v, block_table, k_scale=None, v_scale=None):
        _need(k, "k", 4)
        _need(v, "v", 4)
        _need(block_table, "block_table", 2)
        if k.shape != v.shape or k.dtype != v.dtype:
            raise ValueError("k and v must have the same shape and dtype")
        if block_table.dtype != torch.int32:
            raise TypeError("block_table must be int32")
        if k.dtype == torch.int8:
            for s, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
                _need(s, n, 3)
                if s.dtype != torch.float16 or tuple(s.shape) != tuple(k.shape[:3]):
                    raise ValueError(f"{n} must be float16 of shape {tuple(k.shape[:3])}")
        self.k, self.v, self.block_table = k, v, block_table
        self.k_scale, self.v_scale = k_scale, v_scale
        self.num_pages, self.Hkv, self.page_size, self.d = (int(x) for x in k.shape)

    def _c(self):
        return _PagedKV(self.k.data_ptr(), self.v.data_ptr(),
                        self.k_scale.data_ptr() if self.k_scale is not None else None,
                        self.v_scale.data_ptr() if self.v_scale is not None else None,
                        self.block_table.data_ptr(), self.num_pages, self.page_size, self.Hkv,
                        self.d, int(self.block_table.shape[1]), _dtype_code(self.k, "kv"))


def _shape(t, want, what):
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {devs}")


def _check_batch_kv(batch, kv):
    if int(kv.block_table.shape[0]) != batch.B:
        raise ValueError(f"block_table has {kv.block_table.shape[0]} rows for B = {batch.B}")
    _same_device(batch.ctx_lens, batch.cu_q, kv.k, kv.v, kv.block_table, kv.k_scale, kv.v_scale)


def _check_attn(batch, q, kv, out):
    _need(q, "q", 3)
    _need(out, "out", 3)
    _check_batch_kv(batch, kv)
    if int(q.shape[0]) != batch.total_q or int(q.shape[2]) != kv.d:
        raise ValueError(f"q has shape {tuple(q.shape)}, expected [{batch.total_q}, Hq, {kv.d}]")
    _shape(out, q.shape, "out")
    _same_device(q, out, kv.k)


def _check_append(batch, k_new, v_new, kv):
    _need(k_new, "k_new", 3)
    _need(v_new, "v_new", 3)
    _check_batch_kv(batch, kv)
    _shape(k_new, (batch.total_q, kv.Hkv, kv.d), "k_new")
    _shape(v_new, (batch.total_q, kv.Hkv, kv.d), "v_new")
    if k_new.dtype != v_new.dtype:
        raise TypeError("k_new and v_new must have the same dtype")
    _same_device(k_new, v_new, kv.k)


def _check_accept(batch, logits, draft_ids, argmax_ids, accept_len, next_token):
    _need(logits, "logits", 2)
    _need(draft_ids, "draft_ids", 1)
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    if draft_ids.dtype != torch.int32:
        raise TypeError("draft_ids must be int32")
    if int(logits.shape[0]) != batch.total_q + batch.B:
        raise ValueError(f"logits has {logits.shape[0]} rows, expected T + B = "
                         f"{batch.total_q + batch.B}")
    _shape(draft_ids, (batch.total_q,), "draft_ids")
    for t, n, want in ((argmax_ids, "argmax_ids", batch.total_q + batch.B),
                       (accept_len, "accept_len", batch.B), (next_token, "next_token", batch.B)):
        _need(t, n, 1)
        if t.dtype != torch.int32:
            raise TypeError(f"{n} must be int32")
        _shape(t, (want,), n)
    _same_device(logits, draft_ids, argmax_ids, accept_len, next_token, batch.cu_q)


@_on_stream
def kv_quant_int8(x, codes=None, scales=None, stream=None):
    """INT8 codes and fp16 scales of the rows of x [..., d] (float32 or
    bfloat16).  Returns (codes int8 [..., d], scales float16 [...])."""
    lib = load()
    _need(x, "x")
    d = int(x.shape[-1])
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float16, device=x.device)
    _need(codes, "codes")
    _need(scales, "scales")
    _shape(codes, x.shape, "codes")
    _shape(scales, x.shape[:-1], "scales")
    if codes.dtype != torch.int8 or scales.dtype != torch.float16:
        raise TypeError("codes must be int8 and scales float16")
    _check("sva_kv_quant_int8", lib.sva_kv_quant_int8(
        _ptr(x), _dtype_code(x, "x"), rows, d, _ptr(codes), _ptr(scales),
        _stream(stream, x.device)))
    return codes, scales


@_on_stream
def kv_append(batch, k_new, v_new, kv, stream=None):
    """Write the k_b new rows of every sequence (k_new, v_new [T, Hkv, d]) at
    positions ctx_lens[b] .. ctx_lens[b] + k_b - 1 of the paged cache."""
    lib = load()
    _check_append(batch, k_new, v_new, kv)
    cb, ckv = batch._c(), kv._c()
    _check("sva_kv_append", lib.sva_kv_append(
        ctypes.byref(cb), _ptr(k_new), _ptr(v_new), _dtype_code(k_new, "k_new"),
        ctypes.byref(ckv), _stream(stream, k_new.device)))


def _opts(path, num_workgroups, wait_polls=0):
    return _Opts(int(path), int(num_workgroups), int(wait_polls))


def verify_workspace_bytes(batch, kv, Hq, path=PATH_AUTO, num_workgroups=0):
    lib = load()
    cb, ckv, co = batch._c(), kv._c(), _opts(path, num_workgroups)
    n = lib.sva_verify_workspace_bytes(ctypes.byref(cb), ctypes.byref(ckv), int(Hq),
                                       ctypes.byref(co))
    if n == 0 and batch.total_q > 0:
        raise SvaError("sva_verify_workspace_bytes", 1, lib.sva_last_error().decode())
    return int(n)


_ws_cache = {}


def _zeroed_workspace(device, nbytes):
    """A zero-filled workspace kept per (device, stream) -- the current stream,
    which is the call's (see _on_stream) -- so calls on different streams never
    share counters or partial slots.  The attention kernels leave the counters
    at zero, so it stays reusable in stream order."""
    s = torch.cuda.current_stream(device)
    key = (torch.device(device).index, s.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _check_mask(batch, draft_mask, dev):
    if draft_mask is None:
        return
    _need(draft_mask, "draft_mask", 1)
    if draft_mask.dtype not in (torch.int32, torch.uint32):
        raise TypeError("draft_mask must be int32 or uint32 bit patterns")
    _shape(draft_mask, (batch.total_q,), "draft_mask")
    _same_device(draft_mask, dev)


@_on_stream
def spec_verify_attn(batch, q, kv, softmax_scale=None, out=None, out_dtype=None,
                     workspace=None, path=PATH_AUTO, num_workgroups=0, stream=None,
                     draft_mask=None, wait_polls=0):
    """Verification attention of the drafts q [T, Hq, d] over the paged
    cache: causal among the drafts, or tree attention when draft_mask [T]
    (bit j: draft j of the sequence is visible, see tree_masks) is given.
    Returns out [T, Hq, d] (dtype of q unless out_dtype is given).
    A caller-provided workspace must be zero-filled before its first use."""
    lib = load()
    _need(q, "q", 3)
    Hq, d = int(q.shape[1]), int(q.shape[2])
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _check_attn(batch, q, kv, out)
    _check_mask(batch, draft_mask, q)
    nbytes = verify_workspace_bytes(batch, kv, Hq, path, num_workgroups)
    if workspace is None:
        workspace = _zeroed_workspace(q.device, nbytes)
    _need(workspace, "workspace")
    cb, ckv, co = batch._c(), kv._c(), _opts(path, num_workgroups, wait_polls)
    if draft_mask is None:
        _check("sva_spec_verify_attn", lib.sva_spec_verify_attn(
            ctypes.byref(cb), _ptr(q), _dtype_code(q, "q"), Hq, ctypes.byref(ckv),
            float(softmax_scale), _ptr(out), _dtype_code(out, "out"), ctypes.byref(co),
            _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream, q.device)))
    else:
        _check("sva_spec_verify_attn_tree", lib.sva_spec_verify_attn_tree(
            ctypes.byref(cb), _ptr(q), _dtype_code(q, "q"), Hq, ctypes.byref(ckv),
            _ptr(draft_mask), float(softmax_scale), _ptr(out), _dtype_code(out, "out"),
            ctypes.byref(co), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream, q.device)))
    _debug_check("spec_verify_attn", workspace, stream)
    return out


@_on_stream
def spec_verify_attn_noalloc(batch, q, kv, softmax_scale=None, out=None, out_dtype=None,
                             path=PATH_AUTO, num_workgroups=0, stream=None, wait_polls=0):
    """spec_verify_attn with the library's static scratch as the workspace
    (sva_spec_verify_attn_noalloc: the entry point itself allocates nothing;
    pass `out` to keep this wrapper from allocating it either).  Calls that may
    overlap on one device race on that scratch."""
    lib = load()
    _need(q, "q", 3)
    Hq, d = int(q.shape[1]), int(q.shape[2])
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _check_attn(batch, q, kv, out)
    cb, ckv, co = batch._c(), kv._c(), _opts(path, num_workgroups, wait_polls)
    _check("sva_spec_verify_attn_noalloc", lib.sva_spec_verify_attn_noalloc(
        ctypes.byref(cb), _ptr(q), _dtype_code(q, "q"), Hq, ctypes.byref(ckv),
        float(softmax_scale), _ptr(out), _dtype_code(out, "out"), ctypes.byref(co),
        _stream(stream, q.device)))
    return out


@_on_stream
def spec_verify_attn_append(batch, q, kv, k_new, v_new, softmax_scale=None, out=None,
                            out_dtype=None, workspace=None, path=PATH_AUTO, num_workgroups=0,
                            stream=None, draft_mask=None, wait_polls=0):
    """kv_append(batch, k_new, v_new, kv) then spec_verify_attn(...) in one
    call (one launch on the split-KV kernels): the new rows enter the cache
    and the drafts are verified.  Same results as the two calls."""
    lib = load()
    _need(q, "q", 3)
    Hq, d = int(q.shape[1]), int(q.shape[2])
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _check_append(batch, k_new, v_new, kv)
    _check_attn(batch, q, kv, out)
    _check_mask(batch, draft_mask, q)
    nbytes = verify_workspace_bytes(batch, kv, Hq, path, num_workgroups)
    if workspace is None:
        workspace = _zeroed_workspace(q.device, nbytes)
    _need(workspace, "workspace")
    cb, ckv, co = batch._c(), kv._c(), _opts(path, num_workgroups, wait_polls)
    _check("sva_spec_verify_attn_append", lib.sva_spec_verify_attn_append(
        ctypes.byref(cb), _ptr(q), _dtype_code(q, "q"), Hq, ctypes.byref(ckv), _ptr(k_new),
        _ptr(v_new), _dtype_code(k_new, "k_new"),
        _ptr(draft_mask) if draft_mask is not None else None, float(softmax_scale), _ptr(out),
        _dtype_code(out, "out"), ctypes.byref(co), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, q.device)))
    _debug_check("spec_verify_attn_append", workspace, stream)
    return out


def accept_workspace_bytes(batch, V):
    lib = load()
    cb = batch._c()
    return int(lib.sva_accept_workspace_bytes(ctypes.byref(cb), int(V)))


@_on_stream
def accept_prefix(batch, logits, draft_ids, argmax_ids=None, accept_len=None, next_token=None,
                  workspace=None, stream=None):
    """Greedy longest-prefix acceptance.  logits [T+B, V] float32, draft_ids
    [T] int32.  Returns (argmax_ids [T+B], accept_len [B], next_token [B])."""
    lib = load()
    _need(logits, "logits", 2)
    dev = logits.device
    V = int(logits.shape[1])
    if argmax_ids is None:
        argmax_ids = torch.empty(logits.shape[0], dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(batch.B, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(batch.B, dtype=torch.int32, device=dev)
    _check_accept(batch, logits, draft_ids, argmax_ids, accept_len, next_token)
    if workspace is None:
        workspace = torch.empty(max(accept_workspace_bytes(batch, V), 8), dtype=torch.uint8,
                                device=dev)
    cb = batch._c()
    _check("sva_accept_prefix", lib.sva_accept_prefix(
        ctypes.byref(cb), _ptr(logits), V, _ptr(draft_ids), _ptr(argmax_ids), _ptr(accept_len),
        _ptr(next_token), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream, dev)))
    return argmax_ids, accept_len, next_token


def _int32_vec(t, n, what):
    _need(t, what, 1)
    if t.dtype != torch.int32:
        raise TypeError(f"{what} must be int32")
    _shape(t, (n,), what)


@_on_stream
def tree_masks(batch, parents, masks=None, stream=None):
    """Ancestor bitmasks of token trees: parents [T] int32 (-1: child of the
    last committed token, else an earlier node of the same sequence).
    Returns masks [T] int32 (bit patterns; bit j: node j is the node itself
    or one of its ancestors)."""
    lib = load()
    _int32_vec(parents, batch.total_q, "parents")
    if masks is None:
        masks = torch.empty(batch.total_q, dtype=torch.int32, device=parents.device)
    _int32_vec(masks, batch.total_q, "masks")
    _same_device(parents, masks, batch.cu_q)
    cb = batch._c()
    _check("sva_tree_masks", lib.sva_tree_masks(ctypes.byref(cb), _ptr(parents), _ptr(masks),
                                                _stream(stream, parents.device)))
    return masks


@_on_stream
def accept_tree(batch, logits, draft_ids, parents, argmax_ids=None, accept_len=None,
                next_token=None, accept_path=None, workspace=None, stream=None):
    """Greedy acceptance over token trees.  logits [T+B, V] float32 (row 0 of a
    sequence: after the context, row 1+i: after node i), draft_ids and parents
    [T] int32.  Returns (argmax_ids [T+B], accept_len [B], next_token [B],
    accept_path [T]); accept_path lists each sequence's accepted nodes from the
    root down, then -1."""
    lib = load()
    _need(logits, "logits", 2)
    dev = logits.device
    V = int(logits.shape[1])
    if argmax_ids is None:
        argmax_ids = torch.empty(logits.shape[0], dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(batch.B, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(batch.B, dtype=torch.int32, device=dev)
    if accept_path is None:
        accept_path = torch.empty(batch.total_q, dtype=torch.int32, device=dev)
    _check_accept(batch, logits, draft_ids, argmax_ids, accept_len, next_token)
    _int32_vec(parents, batch.total_q, "parents")
    _int32_vec(accept_path, batch.total_q, "accept_path")
    _same_device(logits, parents, accept_path)
    if workspace is None:
        workspace = torch.empty(max(accept_workspace_bytes(batch, V), 8), dtype=torch.uint8,
                                device=dev)
    cb = batch._c()
    _check("sva_accept_tree", lib.sva_accept_tree(
        ctypes.byref(cb), _ptr(logits), V, _ptr(draft_ids), _ptr(parents), _ptr(argmax_ids),
        _ptr(accept_len), _ptr(next_token), _ptr(accept_path), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, dev)))
    return argmax_ids, accept_len, next_token, accept_path


@_on_stream
def kv_commit_path(batch, accept_len, accept_path, kv, stream=None):
    """Move each sequence's accepted branch (accept_path, from accept_tree) to
    the positions right after its committed context, every kv head."""
    lib = load()
    _int32_vec(accept_len, batch.B, "accept_len")
    _int32_vec(accept_path, batch.total_q, "accept_path")
    _check_batch_kv(batch, kv)
    _same_device(accept_len, accept_path, kv.k)
    cb, ckv = batch._c(), kv._c()
    _check("sva_kv_commit_path", lib.sva_kv_commit_path(
        ctypes.byref(cb), _ptr(accept_len), _ptr(accept_path), ctypes.byref(ckv),
        _stream(stream, kv.k.device)))


def _tree_commit_args(batch, logits, draft_ids, parents, kv, argmax_ids, accept_len,
                      next_token, accept_path, workspace):
    dev = logits.device
    V = int(logits.shape[1])
    if argmax_ids is None:
        argmax_ids = torch.empty(logits.shape[0], dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(batch.B, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(batch.B, dtype=torch.int32, device=dev)
    if accept_path is None:
        accept_path = torch.empty(batch.total_q, dtype=torch.int32, device=dev)
    _check_accept(batch, logits, draft_ids, argmax_ids, accept_len, next_token)
    _int32_vec(parents, batch.total_q, "parents")
    _int32_vec(accept_path, batch.total_q, "accept_path")
    _check_batch_kv(batch, kv)
    _same_device(logits, parents, accept_path, kv.k)
    if workspace is None:
        workspace = torch.empty(max(accept_workspace_bytes(batch, V), 8), dtype=torch.uint8,
                                device=dev)
    cb, ckv = batch._c(), kv._c()
    args = (ctypes.byref(cb), _ptr(logits), V, _ptr(draft_ids), _ptr(parents), ctypes.byref(ckv),
            _ptr(argmax_ids), _ptr(accept_len), _ptr(next_token), _ptr(accept_path),
            _ptr(workspace), workspace.numel() * workspace.element_size())
    keep = (cb, ckv, batch, logits, draft_ids, parents, kv, argmax_ids, accept_len, next_token,
            accept_path, workspace)
    return args, (argmax_ids, accept_len, next_token, accept_path), keep


@_on_stream
def accept_tree_commit(batch, logits, draft_ids, parents, kv, argmax_ids=None, accept_len=None,
                       next_token=None, accept_path=None, workspace=None, stream=None):
    """accept_tree followed by kv_commit_path, in one call (one launch after the
    argmax).  Returns (argmax_ids, accept_len, next_token, accept_path) as
    accept_tree does; the cache ends as kv_commit_path leaves it."""
    lib = load()
    _need(logits, "logits", 2)
    args, outs, _ = _tree_commit_args(batch, logits, draft_ids, parents, kv, argmax_ids,
                                      accept_len, next_token, accept_path, workspace)
    _check("sva_accept_tree_commit",
           lib.sva_accept_tree_commit(*args, _stream(stream, logits.device)))
    return outs


def accept_stochastic_workspace_bytes(batch, V):
    lib = load()
    cb = batch._c()
    return int(lib.sva_accept_stochastic_workspace_bytes(ctypes.byref(cb), int(V)))


def _check_stochastic(batch, target_logits, draft_logits, draft_ids, u_accept, u_sample,
                      accept_len, next_token):
    for t, n, rows in ((target_logits, "target_logits", batch.total_q + batch.B),
                       (draft_logits, "draft_logits", batch.total_q)):
        _need(t, n, 2)
        if t.dtype != torch.float32:
            raise TypeError(f"{n} must be float32")
        if int(t.shape[0]) != rows:
            raise ValueError(f"{n} has {t.shape[0]} rows, expected {rows}")
    if target_logits.shape[1] != draft_logits.shape[1]:
        raise ValueError("target and draft logits must have the same vocabulary")
    _int32_vec(draft_ids, batch.total_q, "draft_ids")
    for t, n, want in ((u_accept, "u_accept", batch.total_q), (u_sample, "u_sample", batch.B)):
        _need(t, n, 1)
        if t.dtype != torch.float32:
            raise TypeError(f"{n} must be float32")
        _shape(t, (want,), n)
    _int32_vec(accept_len, batch.B, "accept_len")
    _int32_vec(next_token, batch.B, "next_token")
    _same_device(target_logits, draft_logits, draft_ids, u_accept, u_sample, accept_len,
                 next_token, batch.cu_q)


@_on_stream
def accept_stochastic(batch, target_logits, draft_logits, draft_ids, u_accept, u_sample,
                      temperature=1.0, accept_len=None, next_token=None, workspace=None,
                      stream=None):
    """Lossless stochastic acceptance.  target_logits [T+B, V] and draft_logits
    [T, V] float32 (p, q = softmax(logits / temperature)), draft_ids [T] int32,
    uniforms u_accept [T] and u_sample [B] float32 in [0, 1).
    Returns (accept_len [B], next_token [B])."""
    lib = load()
    _need(target_logits, "target_logits", 2)
    dev = target_logits.device
    V = int(target_logits.shape[1])
    if accept_len is None:
        accept_len = torch.empty(batch.B, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(batch.B, dtype=torch.int32, device=dev)
    _check_stochastic(batch, target_logits, draft_logits, draft_ids, u_accept, u_sample,
                      accept_len, next_token)
    if workspace is None:
        workspace = torch.empty(max(accept_stochastic_workspace_bytes(batch, V), 256),
                                dtype=torch.uint8, device=dev)
    cb = batch._c()
    _check("sva_accept_stochastic", lib.sva_accept_stochastic(
        ctypes.byref(cb), _ptr(target_logits), _ptr(draft_logits), V, float(temperature),
        _ptr(draft_ids), _ptr(u_accept), _ptr(u_sample), _ptr(accept_len), _ptr(next_token),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, dev)))
    return accept_len, next_token


@_on_stream
def kvmu_apply(state, mode, arg=None, ctx_lens=None, stream=None):
    """Apply KVMU modes to the pointer triplets state [B, 3] int32 (valid,
    curr, ahead) in place.  mode: one KVMU_* value for every sequence, or a
    device [B] int32 tensor of per-sequence modes; arg: device [B] int32 or
    None; ctx_lens: optional device [B] int32 receiving the new valid
    pointers.  Returns state."""
    lib = load()
    _need(state, "state", 2)
    if state.dtype != torch.int32 or int(state.shape[1]) != 3:
        raise ValueError("state must be int32 [B, 3]")
    B = int(state.shape[0])
    per_seq = isinstance(mode, torch.Tensor)
    if per_seq:
        _int32_vec(mode, B, "mode")
    if arg is not None:
        _int32_vec(arg, B, "arg")
    if ctx_lens is not None:
        _int32_vec(ctx_lens, B, "ctx_lens")
    _same_device(state, mode if per_seq else None, arg, ctx_lens)
    _check("sva_kvmu_apply", lib.sva_kvmu_apply(
        B, _ptr(mode) if per_seq else None, 0 if per_seq else int(mode), _ptr(arg), _ptr(state),
        _ptr(ctx_lens), _stream(stream, state.device)))
    return state


def _page_lists(block_table, free_list, free_count):
    _need(block_table, "block_table", 2)
    _need(free_list, "free_list", 1)
    _need(free_count, "free_count", 1)
    for t, n in ((block_table, "block_table"), (free_list, "free_list"),
                 (free_count, "free_count")):
        if t.dtype != torch.int32:
            raise TypeError(f"{n} must be int32")
    if free_count.numel() != 1:
        raise ValueError("free_count must hold one int32")
    _same_device(block_table, free_list, free_count)


@_on_stream
def kv_reclaim_pages(valid_lens, block_table, free_list, free_count, stream=None):
    """Return every page wholly at or past valid_lens[b] (device int32 [B]) of
    block_table [B, max_pages] to the free list (free_list [capacity] int32,
    free_count [1] int32; pages appended after the list's entries) and mark
    its entry -1.  In place, on the device."""
    lib = load()
    _page_lists(block_table, free_list, free_count)
    B = int(block_table.shape[0])
    _int32_vec(valid_lens, B, "valid_lens")
    _same_device(valid_lens, block_table)
    _check("sva_kv_reclaim_pages", lib.sva_kv_reclaim_pages(
        B, _ptr(valid_lens), _ptr(block_table), int(block_table.shape[1]), _ptr(free_list),
        _ptr(free_count), int(free_list.numel()), _stream(stream, block_table.device)))


@_on_stream
def kv_alloc_pages(batch, block_table, free_list, free_count, stream=None):
    """Give every unassigned logical page below S_b + k_b a page from the top
    of the free list (in place, on the device)."""
    lib = load()
    _page_lists(block_table, free_list, free_count)
    if int(block_table.shape[0]) != batch.B:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for B = {batch.B}")
    _same_device(batch.ctx_lens, block_table)
    cb = batch._c()
    _check("sva_kv_alloc_pages", lib.sva_kv_alloc_pages(
        ctypes.byref(cb), _ptr(block_table), int(block_table.shape[1]), _ptr(free_list),
        _ptr(free_count), int(free_list.numel()), _stream(stream, block_table.device)))


@_on_stream
def stream_read_probe(buf, mode=0, num_workgroups=2048, sink=None, stream=None):
    """Read the device buffer `buf` once (its byte size a multiple of 1024)
    with the library's streaming-read probe kernel (mode 0: into registers,
    1: through global -> LDS copies, 2: as 1 over 4 KB pages in a scattered
    order, the byte size 4096 times a power of two).  Returns the sink words."""
    lib = load()
    _need(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(num_workgroups * 4, dtype=torch.int32, device=buf.device)
    _need(sink, "sink", 1)
    if sink.numel() < num_workgroups * 4 or sink.dtype != torch.int32:
        raise ValueError("sink must be int32 with num_workgroups * 4 entries")
    _check("sva_stream_read_probe", lib.sva_stream_read_probe(
        _ptr(buf), nbytes, int(mode), int(num_workgroups), _ptr(sink),
        _stream(stream, buf.device)))
    return sink


class _Prepared:
    """A call with every argument marshalled once; calling it only enqueues
    the C entry point on the stream (current stream of the device by default).
    Workspaces it allocates are filled before it returns (the fill is
    synchronised), so any stream may run the call."""

    def __init__(self, name, fn, args, device, keep, status_ws=None):
        self._name, self._fn, self._args, self._device = name, fn, args, device
        self._keep = keep                        # keeps tensors and structs alive
        self._status_ws = status_ws
        torch.cuda.current_stream(device).synchronize()

    def __call__(self, stream=None):
        _check(self._name, self._fn(*self._args, _stream(stream, self._device)))
        _debug_check(self._name, self._status_ws, stream)


def prepare_kv_append(batch, k_new, v_new, kv):
    lib = load()
    _check_append(batch, k_new, v_new, kv)
    cb, ckv = batch._c(), kv._c()
    args = (ctypes.byref(cb), _ptr(k_new), _ptr(v_new), _dtype_code(k_new, "k_new"),
            ctypes.byref(ckv))
    return _Prepared("sva_kv_append", lib.sva_kv_append, args, k_new.device,
                     (cb, ckv, batch, k_new, v_new, kv))


def prepare_spec_verify_attn(batch, q, kv, out, softmax_scale=None, workspace=None,
                             path=PATH_AUTO, num_workgroups=0, draft_mask=None):
    lib = load()
    _check_attn(batch, q, kv, out)
    _check_mask(batch, draft_mask, q)
    Hq, d = int(q.shape[1]), int(q.shape[2])
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    nbytes = verify_workspace_bytes(batch, kv, Hq, path, num_workgroups)
    if workspace is None:
        workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    cb, ckv, co = batch._c(), kv._c(), _opts(path, num_workgroups)
    if draft_mask is not None:
        args = (ctypes.byref(cb), _ptr(q), _dtype_code(q, "q"), Hq, ctypes.byref(ckv),
                _ptr(draft_mask), float(softmax_scale), _ptr(out), _dtype_code(out, "out"),
                ctypes.byref(co), _ptr(workspace), workspace.numel() * workspace.element_size())
        return _Prepared("sva_spec_verify_attn_tree", lib.sva_spec_verify_attn_tree, args,
                         q.device, (cb, ckv, co, batch, q, kv, out, workspace, draft_mask),
                         workspace)
    args = (ctypes.byref(cb), _ptr(q), _dtype_code(q, "q"), Hq, ctypes.byref(ckv),
            float(softmax_scale), _ptr(out), _dtype_code(out, "out"), ctypes.byref(co),
            _ptr(workspace), workspace.numel() * workspace.element_size())
    return _Prepared("sva_spec_verify_attn", lib.sva_spec_verify_attn, args, q.device,
                     (cb, ckv, co, batch, q, kv, out, workspace), workspace)


def prepare_spec_verify_attn_append(batch, q, kv, k_new, v_new, out, softmax_scale=None,
                                    workspace=None, path=PATH_AUTO, num_workgroups=0,
                                    draft_mask=None):
    lib = load()
    _check_append(batch, k_new, v_new, kv)
    _check_attn(batch, q, kv, out)
    _check_mask(batch, draft_mask, q)
    Hq, d = int(q.shape[1]), int(q.shape[2])
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    nbytes = verify_workspace_bytes(batch, kv, Hq, path, num_workgroups)
    if workspace is None:
        workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    cb, ckv, co = batch._c(), kv._c(), _opts(path, num_workgroups)
    args = (ctypes.byref(cb), _ptr(q), _dtype_code(q, "q"), Hq, ctypes.byref(ckv), _ptr(k_new),
            _ptr(v_new), _dtype_code(k_new, "k_new"),
            _ptr(draft_mask) if draft_mask is not None else None, float(softmax_scale),
            _ptr(out), _dtype_code(out, "out"), ctypes.byref(co), _ptr(workspace),
            workspace.numel() * workspace.element_size())
    return _Prepared("sva_spec_verify_attn_append", lib.sva_spec_verify_attn_append, args,
                     q.device, (cb, ckv, co, batch, q, kv, out, workspace, k_new, v_new,
                                draft_mask), workspace)


def prepare_accept_prefix(batch, logits, draft_ids, argmax_ids, accept_len, next_token,
                          workspace=None):
    lib = load()
    _check_accept(batch, logits, draft_ids, argmax_ids, accept_len, next_token)
    V = int(logits.shape[1])
    if workspace is None:
        workspace = torch.empty(max(accept_workspace_bytes(batch, V), 8), dtype=torch.uint8,
                                device=logits.device)
    cb = batch._c()
    args = (ctypes.byref(cb), _ptr(logits), V, _ptr(draft_ids), _ptr(argmax_ids),
            _ptr(accept_len), _ptr(next_token), _ptr(workspace),
            workspace.numel() * workspace.element_size())
    return _Prepared("sva_accept_prefix", lib.sva_accept_prefix, args, logits.device,
                     (cb, batch, logits, draft_ids, argmax_ids, accept_len, next_token,
                      workspace))


def prepare_tree_masks(batch, parents, masks):
    lib = load()
    _int32_vec(parents, batch.total_q, "parents")
    _int32_vec(masks, batch.total_q, "masks")
    cb = batch._c()
    return _Prepared("sva_tree_masks", lib.sva_tree_masks, (ctypes.byref(cb), _ptr(parents),
                     _ptr(masks)), parents.device, (cb, batch, parents, masks))


def prepare_accept_tree(batch, logits, draft_ids, parents, argmax_ids, accept_len, next_token,
                        accept_path, workspace=None):
    lib = load()
    _check_accept(batch, logits, draft_ids, argmax_ids, accept_len, next_token)
    _int32_vec(parents, batch.total_q, "parents")
    _int32_vec(accept_path, batch.total_q, "accept_path")
    V = int(logits.shape[1])
    if workspace is None:
        workspace = torch.empty(max(accept_workspace_bytes(batch, V), 8), dtype=torch.uint8,
                                device=logits.device)
    cb = batch._c()
    args = (ctypes.byref(cb), _ptr(logits), V, _ptr(draft_ids), _ptr(parents), _ptr(argmax_ids),
            _ptr(accept_len), _ptr(next_token), _ptr(accept_path), _ptr(workspace),
            workspace.numel() * workspace.element_size())
    return _Prepared("sva_accept_tree", lib.sva_accept_tree, args, logits.device,
                     (cb, batch, logits, draft_ids, parents, argmax_ids, accept_len, next_token,
                      accept_path, workspace))


def prepare_kv_commit_path(batch, accept_len, accept_path, kv):
    lib = load()
    _int32_vec(accept_len, batch.B, "accept_len")
    _int32_vec(accept_path, batch.total_q, "accept_path")
    _check_batch_kv(batch, kv)
    cb, ckv = batch._c(), kv._c()
    args = (ctypes.byref(cb), _ptr(accept_len), _ptr(accept_path), ctypes.byref(ckv))
    return _Prepared("sva_kv_commit_path", lib.sva_kv_commit_path, args, kv.k.device,
                     (cb, ckv, batch, accept_len, accept_path, kv))


def prepare_accept_tree_commit(batch, logits, draft_ids, parents, kv, argmax_ids, accept_len,
                               next_token, accept_path, workspace=None):
    lib = load()
    args, _, keep = _tree_commit_args(batch, logits, draft_ids, parents, kv, argmax_ids,
                                      accept_len, next_token, accept_path, workspace)
    return _Prepared("sva_accept_tree_commit", lib.sva_accept_tree_commit, args, logits.device,
                     keep)


def prepare_accept_stochastic(batch, target_logits, draft_logits, draft_ids, u_accept, u_sample,
                              accept_len, next_token, temperature=1.0, workspace=None):
    lib = load()
    _check_stochastic(batch, target_logits, draft_logits, draft_ids, u_accept, u_sample,
                      accept_len, next_token)
    V = int(target_logits.shape[1])
    if workspace is None:
        workspace = torch.empty(max(accept_stochastic_workspace_bytes(batch, V), 256),
                                dtype=torch.uint8, device=target_logits.device)
    cb = batch._c()
    args = (ctypes.byref(cb), _ptr(target_logits), _ptr(draft_logits), V, float(temperature),
            _ptr(draft_ids), _ptr(u_accept), _ptr(u_sample), _ptr(accept_len), _ptr(next_token),
            _ptr(workspace), workspace.numel() * workspace.element_size())
    return _Prepared("sva_accept_stochastic", lib.sva_accept_stochastic, args,
                     target_logits.device, (cb, batch, target_logits, draft_logits, draft_ids,
                                            u_accept, u_sample, accept_len, next_token, workspace))


__all__ += ["prepare_kv_append", "prepare_spec_verify_attn", "prepare_accept_prefix",
            "prepare_accept_stochastic",
            "prepare_tree_masks", "prepare_accept_tree", "prepare_kv_commit_path"]
