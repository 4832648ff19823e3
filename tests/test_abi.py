"""The C ABI library loads and exports every declared entry point; host-checkable
argument errors come back as status codes before anything touches a GPU
(CPU only, no compute calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def _lib():
    import token_verify_attention_amd as tva
    if not os.path.exists(tva.LIB_PATH):
        pytest.skip("library not built")
    return tva, tva.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sva_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_four_operations():
    names = _declared()
    for n in ("sva_spec_verify_attn", "sva_kv_append", "sva_kv_quant_int8", "sva_accept_prefix"):
        assert n in names


def test_library_exports_every_declared_symbol():
    tva, lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    tva, lib = _lib()
    assert lib.sva_status_string(0) == b"SVA_OK"
    assert lib.sva_status_string(1) == b"SVA_ERR_INVALID_ARG"
    assert lib.sva_status_string(2) == b"SVA_ERR_UNSUPPORTED"
    assert lib.sva_status_string(3) == b"SVA_ERR_HIP"


def test_host_checked_errors_need_no_gpu():
    tva, lib = _lib()
    vp = ctypes.c_void_p
    # negative row count, unsupported dtype, unsupported d
    assert lib.sva_kv_quant_int8(vp(16), 0, -1, 128, vp(16), vp(16), None) == 1
    assert lib.sva_kv_quant_int8(vp(16), 3, 4, 128, vp(16), vp(16), None) == 2
    assert lib.sva_kv_quant_int8(vp(16), 0, 4, 96, vp(16), vp(16), None) == 2
    assert b"d = 96" in lib.sva_last_error()
    # zero rows is a no-op that needs no device
    assert lib.sva_kv_quant_int8(None, 0, 0, 128, None, None, None) == 0
    # NULL batch / kv
    assert lib.sva_spec_verify_attn(None, None, 0, 8, None, ctypes.c_float(1.0), None, 0, None,
                                    None, 0, None) == 1
    assert lib.sva_kv_append(None, None, None, 0, None, None) == 1
    assert lib.sva_accept_prefix(None, None, 10, None, None, None, None, None, 0, None) == 1
    # token-tree entry points
    assert lib.sva_tree_masks(None, None, None, None) == 1
    assert lib.sva_spec_verify_attn_tree(None, None, 0, 8, None, None, ctypes.c_float(1.0), None,
                                         0, None, None, 0, None) == 1
    assert lib.sva_accept_tree(None, None, 10, None, None, None, None, None, None, None, 0,
                               None) == 1
    assert lib.sva_kv_commit_path(None, None, None, None, None) == 1
    assert lib.sva_accept_tree_commit(None, None, 10, None, None, None, None, None, None, None,
                                      None, 0, None) == 1
    assert lib.sva_accept_stochastic(None, None, None, 10, ctypes.c_float(1.0), None, None, None,
                                     None, None, None, 0, None) == 1
    # append-and-verify: NULL batch, then NULL new rows and a bad source dtype
    assert lib.sva_spec_verify_attn_append(None, None, 0, 8, None, None, None, 0, None,
                                           ctypes.c_float(1.0), None, 0, None, None, 0, None) == 1
    assert lib.sva_kvmu_apply(-1, None, 0, None, None, None, None) == 1
    assert lib.sva_kvmu_apply(4, None, 9, None, None, None, None) == 1
    assert lib.sva_kvmu_apply(0, None, 1, None, None, None, None) == 0


def test_stream_read_probe_argument_checks():
    tva, lib = _lib()
    vp = ctypes.c_void_p
    assert lib.sva_stream_read_probe(vp(1024), 4096, 3, 256, vp(16), None) == 1      # mode
    assert lib.sva_stream_read_probe(vp(1024), 3 * 4096, 2, 256, vp(16), None) == 1  # 3 pages
    assert b"power of two" in lib.sva_last_error()
    assert lib.sva_stream_read_probe(vp(1024), 1000, 1, 256, vp(16), None) == 1      # not 1 KB
    assert lib.sva_stream_read_probe(vp(1024), 4096, 0, 0, vp(16), None) == 1        # grid
    assert lib.sva_stream_read_probe(None, 0, 2, 256, None, None) == 0               # no bytes


def test_batch_and_cache_shape_checks():
    tva, lib = _lib()
    b = tva._Batch(2, 16, 32, 8, 4, 100)
    kv = tva._PagedKV(16, 32, None, None, 48, 10, 16, 2, 128, 8, tva.SVA_BF16)
    call = lambda Hq, kvs=kv, bs=b: lib.sva_spec_verify_attn(
        ctypes.byref(bs), ctypes.c_void_p(64), 1, Hq, ctypes.byref(kvs), ctypes.c_float(0.1),
        ctypes.c_void_p(64), 1, None, ctypes.c_void_p(64), 1 << 30, None)
    assert call(3) == 1                                    # Hq not a multiple of Hkv
    kv.page_size = 32
    assert call(4) == 2                                    # page size other than 16
    kv.page_size = 16
    kv.d = 96
    assert call(4) == 2                                    # d outside {64, 128}
    kv.d = 128
    kv.kv_dtype = tva.SVA_F32                              # fp32 caches (VALU path):
    b.max_q = 17
    assert call(4) == 2                                    # more than 16 drafts
    b.max_q = 16
    assert call(2 * 64) == 2                               # max_q * G > 128
    kv.kv_dtype = tva.SVA_BF16
    b.B = -1
    assert call(4) == 1
    b.B = 2
    kv.kv_dtype = tva.SVA_INT8                             # INT8 without scales
    assert call(4) == 1
    assert b"scale" in lib.sva_last_error()
    kv.kv_dtype = tva.SVA_F32                              # long steps: MFMA path only
    b.max_q = 64
    assert call(4) == 2
    assert b"MFMA" in lib.sva_last_error()
    b.max_q = 2000                                         # past 1024 drafts
    kv.kv_dtype = tva.SVA_BF16
    assert call(4) == 2
    b.max_q = 16
    kv.kv_dtype = tva.SVA_BF16                             # tree call without its mask
    assert lib.sva_spec_verify_attn_tree(
        ctypes.byref(b), ctypes.c_void_p(64), 1, 4, ctypes.byref(kv), None, ctypes.c_float(0.1),
        ctypes.c_void_p(64), 1, None, ctypes.c_void_p(64), 1 << 30, None) == 1
    assert b"draft_mask" in lib.sva_last_error()
    app = lambda kn, vn, sd: lib.sva_spec_verify_attn_append(    # append and verify
        ctypes.byref(b), ctypes.c_void_p(64), 1, 4, ctypes.byref(kv), kn, vn, sd, None,
        ctypes.c_float(0.1), ctypes.c_void_p(64), 1, None, ctypes.c_void_p(64), 1 << 30, None)
    assert app(None, None, tva.SVA_BF16) == 1
    assert b"k_new" in lib.sva_last_error()
    assert app(ctypes.c_void_p(64), ctypes.c_void_p(64), 3) == 2
    assert app(ctypes.c_void_p(72), ctypes.c_void_p(64), tva.SVA_BF16) == 1   # misaligned


def test_build_flags_keep_ieee_division_and_no_packed_fp32():
    from token_verify_attention_amd import build
    flags = build.compile_flags()
    assert not any("fast-math" in f or "unsafe-fp-math" in f for f in flags)
    assert "-packed-fp32-ops" in flags
    assert "--offload-arch=gfx950" in flags


def test_binding_fails_loudly_without_the_library(monkeypatch):
    import token_verify_attention_amd as tva
    monkeypatch.setattr(tva, "_lib", None)
    monkeypatch.setattr(tva, "LIB_PATH", "/nonexistent/libspecverify.so")
    with pytest.raises(RuntimeError, match="not built"):
        tva.load()


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "token_verify_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f
