"""GPU: sva_spec_verify_attn_noalloc (the workspace is the library's static
scratch) against sva_spec_verify_attn with a workspace argument, through the
C ABI: bit-identical outputs on two calls in a row, the second with a smaller
input, both also within the oracle's tolerance; a shape whose workspace
exceeds the scratch is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import token_verify_attention_amd as tva
from token_verify_attention_amd import workloads as wl
from gpu_helpers import assert_close, batch_of, oracle_attn, paged_kv, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _wk(name, Hq, Hkv, kvd, ident):
    return wl.Workload(name, 1, Hq, Hkv, 128, 0, 1, kvd, "bf16", 0.5 if kvd == "int8" else 1.0,
                       None, None, False, ident)


def _bits(t):
    return t.view(torch.int16)


def _pair(case, nwg):
    batch = batch_of(case)
    kv = paged_kv(case)
    w = case["workload"]
    ref = tva.spec_verify_attn(batch, case["q"], kv, num_workgroups=nwg)
    out = torch.full_like(case["q"], float("nan"))
    tva.spec_verify_attn_noalloc(batch, case["q"], kv, out=out, num_workgroups=nwg)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref))
    kind = "int8" if w.kv_dtype == "int8" else "bf16"
    assert_close(out, oracle_attn(case, quantised=False), kind)
    return out


@pytest.mark.parametrize("kvd", ["bf16", "int8"])
def test_noalloc_equals_workspace_call_on_two_calls(kvd):
    # first a larger batch whose pairs are split over workgroups (partials in
    # the scratch), then a smaller one: stale contents must not leak
    say(f"noalloc {kvd}: large call")
    big = wl.make_case(_wk(f"na-big-{kvd}", 32, 8, kvd, 130), device=DEV,
                       ctx=[3000, 40, 1500, 700, 16], k=[4, 2, 3, 4, 1], with_logits=False)
    _pair(big, 0)
    _pair(big, 40)
    say(f"noalloc {kvd}: smaller call")
    small = wl.make_case(_wk(f"na-small-{kvd}", 16, 4, kvd, 131), device=DEV, ctx=[300, 5],
                         k=[3, 2], with_logits=False)
    _pair(small, 0)
    _pair(small, 7)


def test_noalloc_refuses_shapes_beyond_the_scratch():
    lib = tva.load()
    case = wl.make_case(_wk("na-huge", 32, 8, "bf16", 132), device=DEV, ctx=[2000, 100],
                        k=[16, 3], with_logits=False)
    batch = batch_of(case)
    kv = paged_kv(case)
    out = torch.empty_like(case["q"])
    before = out.clone()
    # 4096 workgroups x 64 query rows per pair need ~270 MB of workspace
    cb, ckv, co = batch._c(), kv._c(), tva._opts(0, 4096)
    st = lib.sva_spec_verify_attn_noalloc(
        ctypes.byref(cb), ctypes.c_void_p(case["q"].data_ptr()), tva.SVA_BF16, 32,
        ctypes.byref(ckv), ctypes.c_float(0.088), ctypes.c_void_p(out.data_ptr()), tva.SVA_BF16,
        ctypes.byref(co), None)
    assert st == tva.SVA_ERR_UNSUPPORTED
    assert b"scratch" in lib.sva_last_error()
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(before))
    # and a call that fits still works afterwards
    small = torch.empty_like(case["q"])
    tva.spec_verify_attn_noalloc(batch, case["q"], kv, out=small)
    torch.cuda.synchronize()
    assert_close(small, oracle_attn(case), "bf16")
