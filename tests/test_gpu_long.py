"""GPU parity of verification attention with long speculated steps (through
the C ABI): tens to hundreds of drafts per sequence, as when a process reward
model scores a whole reasoning step in one pass ("HeteroReason").  These
shapes run on the row-block kernel (256 query rows per workgroup, pages shared
by its eight waves).  Small cases cover k from 17 to 300, GQA groups 1 to 7,
bf16 and INT8 caches, d = 64 / 128, S = 0 and ragged mixes; tree masks with
more than 128 rows per pair take the same kernel (every cache type and d);
the full prm7b_step workload is checked on sampled pairs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import token_verify_attention_amd as tva
from token_verify_attention_amd import workloads as wl
from gpu_helpers import assert_close, batch_of, np_, oracle_attn, paged_kv, rows_of_pairs, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W = wl.Workload


def _wk(name, Hq, Hkv, d, kv, q, sigma=1.0, ident=110):
    return W(name, 1, Hq, Hkv, d, 0, 1, kv, q, sigma, None, None, False, ident)


LONG = [
    (_wk("long-bf16-g7", 28, 4, 128, "bf16", "bf16", ident=111), [500, 0, 63], [128, 40, 17]),
    (_wk("long-bf16-mha", 8, 8, 128, "bf16", "bf16", ident=112), [16, 300], [300, 129]),
    (_wk("long-int8-g4", 16, 4, 128, "int8", "bf16", 0.5, ident=113), [200, 1], [64, 100]),
    (_wk("long-bf16-d64", 8, 2, 64, "bf16", "bf16", ident=114), [31, 700, 5], [33, 96, 250]),
    (_wk("long-mixed", 16, 4, 128, "bf16", "bf16", ident=115), [90, 10, 1000, 0], [4, 150, 1, 64]),
]


@pytest.mark.parametrize("spec", LONG, ids=[s[0].name for s in LONG])
def test_long_steps(spec):
    w, ctx, ks = spec
    say(f"long steps {w.name}")
    case = wl.make_case(w, device=DEV, ctx=ctx, k=ks, with_logits=False)
    kv = paged_kv(case)
    out = tva.spec_verify_attn(batch_of(case), case["q"], kv)
    torch.cuda.synchronize()
    if w.kv_dtype == "int8":
        assert_close(out, oracle_attn(case, quantised=True), "int8_deq")
        assert_close(out, oracle_attn(case, quantised=False), "int8")
    else:
        assert_close(out, oracle_attn(case), "bf16")


def test_long_steps_after_append():
    """The k new rows appended by sva_kv_append are the drafts attention reads."""
    w = _wk("long-append", 28, 4, 128, "bf16", "bf16", ident=116)
    case = wl.make_case(w, device=DEV, ctx=[100, 7], k=[128, 200], with_logits=False)
    batch = batch_of(case)
    kv = paged_kv(case)
    tva.kv_append(batch, case["k_new"], case["v_new"], kv)
    out = tva.spec_verify_attn(batch, case["q"], kv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.spec_verify_attn(np_(case["q"]), np_(kv.k), np_(kv.v), np_(case["block_table"]),
                                  np_(case["ctx_lens"]), np_(case["cu_q"]), 1.0 / math.sqrt(w.d))
    assert_close(out, ref, "bf16")


def test_tree_mask_on_row_block_kernel():
    """16 tree nodes x G = 16: 256 query rows per pair, beyond the split kernel."""
    w = _wk("long-tree", 64, 4, 128, "bf16", "bf16", ident=117)
    ks = [16, 9, 16]
    case = wl.make_case(w, device=DEV, ctx=[70, 0, 300], k=ks, with_logits=False)
    parents = wl.make_tree(ks, device=DEV, seed=3)
    batch = batch_of(case)
    masks = tva.tree_masks(batch, parents)
    out = tva.spec_verify_attn(batch, case["q"], paged_kv(case), draft_mask=masks)
    torch.cuda.synchronize()
    om = oracle.ancestor_masks(np_(parents), np_(case["cu_q"]))
    ref = oracle.spec_verify_attn(np_(case["q"]), np_(case["k_pool"]), np_(case["v_pool"]),
                                  np_(case["block_table"]), np_(case["ctx_lens"]),
                                  np_(case["cu_q"]), 1.0 / math.sqrt(w.d), draft_mask=om)
    assert_close(out, ref, "bf16")


# The row-block kernel's remaining instantiations (cache type x d x mask form)
# beyond the cases above: INT8 at d = 64 (causal), tree masks on INT8 and
# d = 64 caches (16 nodes x G = 16: 256 rows per pair), and both ways a block
# copies its pages: 256-row blocks (every wave holds rows: one page per
# second-half wave) and 224-row blocks (the last wave holds none and copies
# every page), on bf16 and INT8 caches with many committed groups.  These
# shapes take the row-block kernel by rule (more than 16 drafts or 128 rows
# per pair); on a 256-CU part rows-int8-d64 and rows-int8-tree cut their
# blocks into 2 key slices and the INT8 copy cases into 3, the others (fewer
# page groups per block) keep one.
ROW_VARIANTS = [
    (_wk("rows-int8-d64", 16, 4, 64, "int8", "bf16", 0.5, ident=119), [300, 5], [40, 70], False),
    (_wk("rows-int8-tree", 64, 4, 128, "int8", "bf16", 0.5, ident=120), [70, 0, 300], [16, 9, 16],
     True),
    (_wk("rows-d64-tree", 64, 4, 64, "bf16", "bf16", ident=121), [70, 3, 300], [16, 12, 16], True),
    (_wk("rows-int8-d64-tree", 64, 4, 64, "int8", "bf16", 0.5, ident=122), [33, 0, 200],
     [16, 16, 5], True),
    (_wk("copy-bf16-256rows", 16, 4, 128, "bf16", "bf16", ident=123), [300, 170], [64, 64], False),
    (_wk("copy-bf16-224rows", 16, 4, 128, "bf16", "bf16", ident=124), [300, 170], [56, 56], False),
    (_wk("copy-int8-256rows", 16, 4, 128, "int8", "bf16", 0.5, ident=125), [300, 170], [64, 64],
     False),
    (_wk("copy-int8-224rows", 16, 4, 128, "int8", "bf16", 0.5, ident=126), [300, 170], [56, 56],
     False),
]


@pytest.mark.parametrize("spec", ROW_VARIANTS, ids=[s[0].name for s in ROW_VARIANTS])
def test_row_block_kernel_variants(spec):
    w, ctx, ks, tree = spec
    say(f"row-block variant {w.name}")
    case = wl.make_case(w, device=DEV, ctx=ctx, k=ks, with_logits=False)
    batch = batch_of(case)
    kv = paged_kv(case)
    om = None
    if tree:
        parents = wl.make_tree(ks, device=DEV, seed=w.ident)
        out = tva.spec_verify_attn(batch, case["q"], kv, draft_mask=tva.tree_masks(batch, parents))
        om = oracle.ancestor_masks(np_(parents), np_(case["cu_q"]))
    else:
        out = tva.spec_verify_attn(batch, case["q"], kv)
    torch.cuda.synchronize()
    qn, kp, vp = np_(case["q"]), np_(case["k_pool"]), np_(case["v_pool"])
    args = (np_(case["block_table"]), np_(case["ctx_lens"]), np_(case["cu_q"]), 1.0 / math.sqrt(w.d))
    if w.kv_dtype == "int8":
        P, H = kp.shape[:2]
        kc, ksc = oracle.kv_quant_int8(kp.reshape(-1, w.d))
        vc, vsc = oracle.kv_quant_int8(vp.reshape(-1, w.d))
        ref_q = oracle.spec_verify_attn(qn, kc.reshape(kp.shape), vc.reshape(vp.shape), *args,
                                        k_scale=ksc.reshape(P, H, 16), v_scale=vsc.reshape(P, H, 16),
                                        draft_mask=om)
        assert_close(out, ref_q, "int8_deq")
        assert_close(out, oracle.spec_verify_attn(qn, kp, vp, *args, draft_mask=om), "int8")
    else:
        assert_close(out, oracle.spec_verify_attn(qn, kp, vp, *args, draft_mask=om), "bf16")


def test_row_block_kernel_equals_split_kernel_on_short_steps():
    """Sequences both kernels take (k*G = 64 and 48 rows per pair).  In a batch
    of 128 such sequences the row blocks fill the device and the row-block
    kernel runs (its workspace is the counters alone); the first two of them
    as a batch of their own run on the split kernel.  Both agree with the
    oracle, and with each other within the bar."""
    w = _wk("both", 16, 4, 128, "bf16", "bf16", ident=118)
    case = wl.make_case(w, device=DEV, ctx=[400, 33] * 64, k=[16, 12] * 64, with_logits=False)
    kv = paged_kv(case)
    big = batch_of(case)
    assert tva.verify_workspace_bytes(big, kv, w.Hq) == tva.STATUS_OFFSET + 256   # row blocks
    rows_out = tva.spec_verify_attn(big, case["q"], kv, out_dtype=torch.float32)
    t2 = 16 + 12                                     # the first two sequences' drafts
    small = tva.Batch(case["ctx_lens"][:2].contiguous(), case["cu_q"][:3].contiguous(),
                      total_q=t2, max_q=16, max_len=416)
    kv2 = tva.PagedKV(kv.k, kv.v, case["block_table"][:2].contiguous())
    assert tva.verify_workspace_bytes(small, kv2, w.Hq) > tva.STATUS_OFFSET + 256   # split
    split_out = tva.spec_verify_attn(small, case["q"][:t2].contiguous(), kv2,
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    pairs = [(b, g) for b in range(2) for g in range(w.Hkv)]
    ref = oracle_attn(case, select=pairs)[:t2]
    assert_close(rows_out[:t2], ref, "bf16")
    assert_close(split_out, ref, "bf16")
    assert_close(split_out, np_(rows_out[:t2]).astype(np.float64), "bf16")


def test_prm7b_step_full_size_sampled():
    w = wl.WORKLOADS["prm7b_step"]
    say("prm7b_step full size")
    case = wl.make_case(w, device=DEV, with_logits=False)
    kv = paged_kv(case)
    out = tva.spec_verify_attn(batch_of(case), case["q"], kv)
    torch.cuda.synchronize()
    pairs = [(0, 0), (5, 3), (11, 1), (15, 2)]
    ref = oracle_attn(case, select=pairs)
    assert_close(out, ref, "bf16", rows=rows_of_pairs(case, pairs))


# One sequence of the 7B PRM shape: its 4 pairs of 896 query rows make 16 row
# blocks, far fewer than the CUs, so each block's keys are cut into slices
# streamed by separate workgroups whose partial states a second launch folds
# (the workspace then holds those states).  Checked on every query row.
KEY_SLICES = [
    (_wk("slices-bf16", 28, 4, 128, "bf16", "bf16", ident=127), [3000], [128], False),
    (_wk("slices-int8", 28, 4, 128, "int8", "bf16", 0.5, ident=128), [2100], [128], False),
    (_wk("slices-d64-two", 16, 4, 64, "bf16", "bf16", ident=129), [1500, 40], [96, 200], False),
    (_wk("slices-tree", 64, 4, 128, "bf16", "bf16", ident=130), [2000], [16], True),
]


@pytest.mark.parametrize("spec", KEY_SLICES, ids=[s[0].name for s in KEY_SLICES])
def test_row_blocks_cut_into_key_slices(spec):
    w, ctx, ks, tree = spec
    say(f"row-block key slices {w.name}")
    case = wl.make_case(w, device=DEV, ctx=ctx, k=ks, with_logits=False)
    batch = batch_of(case)
    kv = paged_kv(case)
    assert tva.verify_workspace_bytes(batch, kv, w.Hq) > tva.STATUS_OFFSET + 256   # sliced
    masks = om = None
    if tree:
        parents = wl.make_tree(ks, device=DEV, seed=w.ident)
        masks = tva.tree_masks(batch, parents)
        om = oracle.ancestor_masks(np_(parents), np_(case["cu_q"]))
    out = tva.spec_verify_attn(batch, case["q"], kv, draft_mask=masks)
    again = tva.spec_verify_attn(batch, case["q"], kv, draft_mask=masks)
    torch.cuda.synchronize()
    assert torch.equal(out, again)                     # the slices fold in a fixed order
    qn, kp, vp = np_(case["q"]), np_(case["k_pool"]), np_(case["v_pool"])
    args = (np_(case["block_table"]), np_(case["ctx_lens"]), np_(case["cu_q"]), 1.0 / math.sqrt(w.d))
    if w.kv_dtype == "int8":
        P, H = kp.shape[:2]
        kc, ksc = oracle.kv_quant_int8(kp.reshape(-1, w.d))
        vc, vsc = oracle.kv_quant_int8(vp.reshape(-1, w.d))
        ref_q = oracle.spec_verify_attn(qn, kc.reshape(kp.shape), vc.reshape(vp.shape), *args,
                                        k_scale=ksc.reshape(P, H, 16), v_scale=vsc.reshape(P, H, 16))
        assert_close(out, ref_q, "int8_deq")
        assert_close(out, oracle.spec_verify_attn(qn, kp, vp, *args), "int8")
    else:
        assert_close(out, oracle.spec_verify_attn(qn, kp, vp, *args, draft_mask=om), "bf16")


def test_key_slices_without_allocation():
    """The allocation-free entry point limits the slices' partial states to its
    static scratch (fewer slices) and gives the same rows within the bar."""
    w = KEY_SLICES[0][0]
    case = wl.make_case(w, device=DEV, ctx=[3000], k=[128], with_logits=False)
    batch = batch_of(case)
    kv = paged_kv(case)
    out = tva.spec_verify_attn_noalloc(batch, case["q"], kv)
    torch.cuda.synchronize()
    ref = oracle.spec_verify_attn(np_(case["q"]), np_(case["k_pool"]), np_(case["v_pool"]),
                                  np_(case["block_table"]), np_(case["ctx_lens"]),
                                  np_(case["cu_q"]), 1.0 / math.sqrt(w.d))
    assert_close(out, ref, "bf16")


def test_prm7b_step_b1_full_size_every_pair():
    """One sequence of the 7B PRM shape (its row blocks cut into key slices),
    through the fused append call the benchmark times, on every pair."""
    w = wl.WORKLOADS["prm7b_step_b1"]
    say("prm7b_step_b1 full size")
    case = wl.make_case(w, device=DEV, with_logits=False)
    batch = batch_of(case)
    kv = paged_kv(case)
    kp, vp = np_(case["k_pool"]), np_(case["v_pool"])          # before the GPU append
    out = tva.spec_verify_attn_append(batch, case["q"], kv, case["k_new"], case["v_new"])
    torch.cuda.synchronize()
    bt, ctx, cu = np_(case["block_table"]), np_(case["ctx_lens"]), np_(case["cu_q"])
    kp, vp, _, _ = oracle.kv_append(np_(case["k_new"]), np_(case["v_new"]), kp, vp, bt, ctx, cu,
                                    "bf16")
    ref = oracle.spec_verify_attn(np_(case["q"]), kp, vp, bt, ctx, cu, 1.0 / math.sqrt(w.d))
    assert_close(out, ref, "bf16")


# bf16 pairs of 33-128 query rows whose query heads cannot be split into one
# 32-row pass (odd G) take the row-block kernel, cut into key slices here.
MULTI_PASS = [
    (_wk("g7-56rows", 28, 4, 128, "bf16", "bf16", ident=131), [300, 1000, 40, 0], [8, 5, 8, 3]),
    (_wk("g3-48rows", 24, 8, 128, "bf16", "bf16", ident=132), [500, 77], [16, 9]),
]


@pytest.mark.parametrize("spec", MULTI_PASS, ids=[s[0].name for s in MULTI_PASS])
def test_multi_pass_pairs_on_row_blocks(spec):
    w, ctx, ks = spec
    say(f"multi-pass pairs {w.name}")
    case = wl.make_case(w, device=DEV, ctx=ctx, k=ks, with_logits=False)
    out = tva.spec_verify_attn(batch_of(case), case["q"], paged_kv(case))
    torch.cuda.synchronize()
    assert_close(out, oracle_attn(case), "bf16")
