"""GPU: sva_spec_verify_attn_append equals sva_kv_append followed by
sva_spec_verify_attn (or its tree variant) on the same inputs -- the same
cache bytes and bit-identical outputs (through the C ABI).

Covered: bf16 and INT8 caches, fp32 and bf16 new rows, d = 64 / 128, ragged
contexts (S = 0, page-boundary and mid-page draft rows), grids that split a
pair's draft pages over workgroups, token trees, long speculated steps (the
row-block kernel appends in a launch of its own) and the benchmark's full
8B-GQA and 70B-INT8 shapes.  One case is also checked against the oracle
(append, then attention).
"""
import numpy as np
import pytest
import torch

import oracle
import token_verify_attention_amd as tva
from token_verify_attention_amd import workloads as wl
from gpu_helpers import assert_close, batch_of, np_, quantise_pool, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _wk(name, Hq, Hkv, d, kvd, ident):
    q = "bf16"
    return wl.Workload(name, 1, Hq, Hkv, d, 0, 1, kvd, q, 0.5 if kvd == "int8" else 1.0, None,
                       None, True, ident)


def _two_caches(case, kvd):
    """Two independent copies of the case's cache in its stored format."""
    if kvd == "int8":
        kc, ks = quantise_pool(case["k_pool"])
        vc, vs = quantise_pool(case["v_pool"])
        mk = lambda: tva.PagedKV(kc.clone(), vc.clone(), case["block_table"], ks.clone(),
                                 vs.clone())
    else:
        dt = torch.float32 if kvd == "f32" else torch.bfloat16
        k, v = case["k_pool"].to(dt), case["v_pool"].to(dt)
        mk = lambda: tva.PagedKV(k.clone(), v.clone(), case["block_table"])
    return mk(), mk()


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int8 if t.element_size() == 1 else torch.int32)


def _same_cache(a, b):
    assert torch.equal(_bits(a.k), _bits(b.k)) and torch.equal(_bits(a.v), _bits(b.v))
    if a.k_scale is not None:
        assert torch.equal(_bits(a.k_scale), _bits(b.k_scale))
        assert torch.equal(_bits(a.v_scale), _bits(b.v_scale))


def _compare(case, kvd, src="f32", nwg=0, mask=None):
    kv_a, kv_b = _two_caches(case, kvd)
    kn, vn = case["k_new"], case["v_new"]
    if src == "bf16":
        kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    else:
        kn, vn = kn.float(), vn.float()
    b = batch_of(case)
    tva.kv_append(b, kn, vn, kv_a)
    out_a = tva.spec_verify_attn(b, case["q"], kv_a, num_workgroups=nwg, draft_mask=mask)
    out_b = tva.spec_verify_attn_append(b, case["q"], kv_b, kn, vn, num_workgroups=nwg,
                                        draft_mask=mask)
    torch.cuda.synchronize()
    _same_cache(kv_a, kv_b)
    assert torch.equal(_bits(out_a), _bits(out_b))
    assert torch.isfinite(out_b.float()).all()
    return out_b, kv_b, kn, vn


CTX = [0, 1, 15, 16, 17, 100, 300]
KS = [4, 1, 3, 4, 2, 4, 4]


@pytest.mark.parametrize("kvd", ["bf16", "int8"])
@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("nwg", [0, 3, 64])
def test_fused_equals_append_then_attention(kvd, src, nwg):
    say(f"fused append {kvd} src={src} nwg={nwg}")
    w = _wk(f"fa-{kvd}", 16, 4, 128, kvd, ident=120)
    case = wl.make_case(w, device=DEV, ctx=CTX, k=KS, with_logits=False)
    _compare(case, kvd, src, nwg)


@pytest.mark.parametrize("kvd", ["bf16", "int8"])
def test_fused_d64_and_draft_pages_split_over_workgroups(kvd):
    """d = 64, and drafts straddling a page boundary with a grid large enough
    to cut draft pages of one pair over different workgroups."""
    w = _wk(f"fa64-{kvd}", 8, 2, 64, kvd, ident=121)
    case = wl.make_case(w, device=DEV, ctx=[30, 47, 2, 61], k=[16, 9, 5, 16], with_logits=False)
    for nwg in (1, 7, 40):
        _compare(case, kvd, "f32", nwg)


def test_fused_tree_step():
    w = _wk("fa-tree", 16, 4, 128, "bf16", ident=122)
    ks = [8, 5, 1, 8]
    case = wl.make_case(w, device=DEV, ctx=[40, 300, 0, 17], k=ks, with_logits=False)
    parents = wl.make_tree(ks, device=DEV, seed=3)
    mask = tva.tree_masks(batch_of(case), parents)
    _compare(case, "bf16", "bf16", 0, mask)


def test_fused_long_steps_take_the_separate_append():
    w = _wk("fa-long", 16, 2, 128, "bf16", ident=123)
    case = wl.make_case(w, device=DEV, ctx=[200, 33], k=[64, 100], with_logits=False)
    _compare(case, "bf16", "bf16", 0)


def test_fused_against_the_oracle():
    """Append then attention in fp64 (oracle) against the fused call."""
    w = _wk("fa-oracle", 16, 4, 128, "bf16", ident=124)
    case = wl.make_case(w, device=DEV, ctx=CTX, k=KS, with_logits=False)
    kp, vp = np_(case["k_pool"].to(torch.bfloat16)), np_(case["v_pool"].to(torch.bfloat16))
    out, _, kn, vn = _compare(case, "bf16", "bf16", 0)
    bt, ctx, cu = np_(case["block_table"]), np_(case["ctx_lens"]), np_(case["cu_q"])
    kp, vp, _, _ = oracle.kv_append(np_(kn), np_(vn), kp, vp, bt, ctx, cu, "bf16")
    ref = oracle.spec_verify_attn(np_(case["q"]), kp, vp, bt, ctx, cu, 1.0 / np.sqrt(w.d))
    assert_close(out, ref, "bf16")


# gqa70b_int8_tp8 (16 pairs of 32 query rows) splits each kv head's query
# heads over two workgroups, so its fused call appends in a launch of its own
@pytest.mark.parametrize("name", ["gqa8b", "gqa70b_int8", "gqa70b_int8_tp8"])
def test_fused_full_size(name):
    w = wl.WORKLOADS[name]
    say(f"fused append full size {name}")
    case = wl.make_case(w, device=DEV, with_logits=False)
    _compare(case, w.kv_dtype, "f32" if w.kv_dtype == "int8" else "bf16", 0)
