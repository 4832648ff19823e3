"""GPU parity of the token-tree entry points against the fp64 oracle (through
the C ABI): sva_tree_masks (bit-exact), sva_spec_verify_attn_tree (stated
tolerances; a chain tree reproduces the causal call bitwise), sva_accept_tree
(bit-exact argmax, lengths, tokens and paths) and sva_kv_commit_path
(bit-exact pools, INT8 scales included).  Small cases cover every tree shape
the generator draws, invalid parents, S = 0, ragged k and split pairs; the
full tree8b workload is checked on sampled (sequence, kv-head) pairs.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import token_verify_attention_amd as tva
from token_verify_attention_amd import workloads as wl
from gpu_helpers import assert_close, batch_of, np_, paged_kv, rows_of_pairs, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W = wl.Workload


def _wk(name, Hq, Hkv, d, kv, q, sigma=1.0, ident=70, vocab=None, match=None):
    return W(name, 1, Hq, Hkv, d, 0, 1, kv, q, sigma, vocab, match, False, ident)


def _masks_oracle(case, parents):
    return oracle.ancestor_masks(np_(parents), np_(case["cu_q"]))


def test_masks_bit_exact_incl_invalid_parents():
    for seed in range(4):
        ks = [16, 1, 0, 7, 12, 3]
        ctx = [10] * len(ks)
        case = wl.make_case(_wk("m", 4, 4, 64, "f32", "f32"), device=DEV, ctx=ctx, k=ks,
                            with_logits=False)
        parents = wl.make_tree(ks, device=DEV, seed=seed)
        if seed == 3:                       # out-of-range parents read as roots
            parents[3] = 7
            parents[5] = -9
            parents[20] = 100
        say(f"tree masks seed={seed}")
        got = tva.tree_masks(batch_of(case), parents)
        torch.cuda.synchronize()
        want = _masks_oracle(case, parents)
        assert np.array_equal(np_(got).astype(np.uint32), want.astype(np.uint32))


ATTN = [
    (_wk("tree-bf16-gqa4", 16, 4, 128, "bf16", "bf16", ident=71), [0, 1, 17, 100, 260], [16, 8, 5, 1, 8]),
    (_wk("tree-bf16-mha", 8, 8, 128, "bf16", "bf16", ident=72), [31, 5, 64], [12, 16, 3]),
    (_wk("tree-int8-gqa8", 32, 4, 128, "int8", "bf16", 0.5, ident=73), [200, 17, 3], [4, 3, 2]),
    (_wk("tree-f32-d64", 4, 4, 64, "f32", "f32", ident=74), [128, 40, 0], [8, 3, 6]),
    (_wk("tree-bf16-d64", 8, 2, 64, "bf16", "bf16", ident=75), [70, 1, 33], [16, 8, 2]),
]


def _oracle_tree(case, masks, quantised=True):
    w = case["workload"]
    kp, vp = np_(case["k_pool"]), np_(case["v_pool"])
    args = {}
    if w.kv_dtype == "int8" and quantised:
        P, H = kp.shape[:2]
        kc, ks = oracle.kv_quant_int8(kp.reshape(-1, w.d))
        vc, vs = oracle.kv_quant_int8(vp.reshape(-1, w.d))
        kp, vp = kc.reshape(kp.shape), vc.reshape(vp.shape)
        args.update(k_scale=ks.reshape(P, H, 16), v_scale=vs.reshape(P, H, 16))
    return oracle.spec_verify_attn(np_(case["q"]), kp, vp, np_(case["block_table"]),
                                   np_(case["ctx_lens"]), np_(case["cu_q"]), 1.0 / math.sqrt(w.d),
                                   draft_mask=masks, **args)


@pytest.mark.parametrize("path", [0, 1], ids=["auto", "valu"])
@pytest.mark.parametrize("spec", ATTN, ids=[s[0].name for s in ATTN])
def test_tree_attention(spec, path):
    w, ctx, ks = spec
    say(f"tree attn {w.name} path={path}")
    case = wl.make_case(w, device=DEV, ctx=ctx, k=ks, with_logits=False)
    parents = wl.make_tree(ks, device=DEV, seed=w.ident)
    batch = batch_of(case)
    masks = tva.tree_masks(batch, parents)
    kv = paged_kv(case)
    out = tva.spec_verify_attn(batch, case["q"], kv, path=path, draft_mask=masks)
    torch.cuda.synchronize()
    om = _masks_oracle(case, parents)
    if w.kv_dtype == "int8":
        assert_close(out, _oracle_tree(case, om, quantised=True), "int8_deq")
        assert_close(out, _oracle_tree(case, om, quantised=False), "int8")
    else:
        assert_close(out, _oracle_tree(case, om), "f32" if w.kv_dtype == "f32" else "bf16")


@pytest.mark.parametrize("nwg", [1, 3, 64, 300])
def test_tree_attention_split_pairs(nwg):
    w = _wk("tree-split", 16, 4, 128, "bf16", "bf16", ident=76)
    ks = [16, 8, 3, 16]
    case = wl.make_case(w, device=DEV, ctx=[700, 33, 1, 260], k=ks, with_logits=False)
    parents = wl.make_tree(ks, device=DEV, seed=5)
    batch = batch_of(case)
    say(f"tree attn split W={nwg}")
    out = tva.spec_verify_attn(batch, case["q"], paged_kv(case), num_workgroups=nwg,
                               draft_mask=tva.tree_masks(batch, parents))
    torch.cuda.synchronize()
    assert_close(out, _oracle_tree(case, _masks_oracle(case, parents)), "bf16")


@pytest.mark.parametrize("kvd", ["bf16", "int8", "f32"])
def test_chain_tree_reproduces_causal_bitwise(kvd):
    w = _wk(f"chain-{kvd}", 16, 4, 128 if kvd != "f32" else 64, kvd,
            "bf16" if kvd != "f32" else "f32", 0.5 if kvd == "int8" else 1.0, ident=77)
    ks = [4, 16, 1, 9]
    case = wl.make_case(w, device=DEV, ctx=[50, 300, 0, 17], k=ks, with_logits=False)
    chain = torch.tensor([i - 1 for k in ks for i in range(k)], dtype=torch.int32, device=DEV)
    batch = batch_of(case)
    kv = paged_kv(case)
    say(f"chain tree {kvd}")
    a = tva.spec_verify_attn(batch, case["q"], kv)
    b = tva.spec_verify_attn(batch, case["q"], kv, draft_mask=tva.tree_masks(batch, chain))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _accept_case(ks, V, match, seed, ident):
    w = _wk("acc", 4, 4, 64, "f32", "f32", ident=ident, vocab=V, match=match)
    case = wl.make_case(w, device=DEV, ctx=[5] * len(ks), k=ks, with_logits=False)
    parents = wl.make_tree(ks, device=DEV, seed=seed)
    case.update(wl.make_tree_logits(w, ks, parents, device=DEV))
    return case, parents


@pytest.mark.parametrize("V,match", [(1000, 0.8), (128256, 0.9), (37, 0.5), (4099, 1.0)])
def test_tree_acceptance_bit_exact(V, match):
    ks = [16, 8, 1, 0, 5, 16, 2]
    case, parents = _accept_case(ks, V, match, seed=V % 97, ident=78)
    say(f"tree accept V={V} p={match}")
    ids, n, nxt, path = tva.accept_tree(batch_of(case), case["logits"], case["draft_ids"], parents)
    torch.cuda.synchronize()
    rt, rn, rx, rp = oracle.accept_tree(np_(case["logits"]), np_(case["draft_ids"]), np_(parents),
                                        np_(case["cu_q"]))
    assert np.array_equal(np_(ids), rt)
    assert np.array_equal(np_(n), rn)
    assert np.array_equal(np_(nxt), rx)
    assert np.array_equal(np_(path), rp)
    if match == 1.0:
        assert (rn > 0).sum() == sum(1 for k in ks if k)


def test_tree_acceptance_ties_and_duplicates():
    """Tied maxima (lowest index wins) and sibling nodes carrying the same token."""
    ks = [6]
    case, _ = _accept_case(ks, 64, 0.0, seed=1, ident=79)
    logits = torch.zeros(7, 64, device=DEV)
    logits[0, [9, 3]] = 2.0                # tie: token 3
    logits[1, 5] = 1.0
    logits[2, 8] = float("nan")             # NaN counts as the maximum
    # root row -> token 3 (tie 3/9) -> node 1; node 1's row -> 8 (NaN) -> node 2
    # (node 5 also carries 8: the lower index wins); node 2's row (all zero)
    # -> 0 -> node 3; node 3 has no children: n = 3, next token 0
    parents = torch.tensor([-1, -1, 1, 2, 0, 1], dtype=torch.int32, device=DEV)
    drafts = torch.tensor([7, 3, 8, 0, 5, 8], dtype=torch.int32, device=DEV)
    ids, n, nxt, path = tva.accept_tree(batch_of(case), logits, drafts, parents)
    torch.cuda.synchronize()
    rt, rn, rx, rp = oracle.accept_tree(np_(logits), np_(drafts), np_(parents), np_(case["cu_q"]))
    assert np.array_equal(np_(ids), rt) and np.array_equal(np_(n), rn)
    assert np.array_equal(np_(nxt), rx) and np.array_equal(np_(path), rp)
    assert int(n[0]) == 3 and list(np_(path)[:3]) == [1, 2, 3] and int(nxt[0]) == 0


def test_chain_tree_acceptance_equals_prefix():
    ks = [4, 8, 1, 16, 3]
    w = _wk("chainacc", 4, 4, 64, "f32", "f32", ident=80, vocab=5000, match=0.8)
    case = wl.make_case(w, device=DEV, ctx=[5] * len(ks), k=ks)
    chain = torch.tensor([i - 1 for k in ks for i in range(k)], dtype=torch.int32, device=DEV)
    batch = batch_of(case)
    a = tva.accept_prefix(batch, case["logits"], case["draft_ids"])
    b = tva.accept_tree(batch, case["logits"], case["draft_ids"], chain)
    torch.cuda.synchronize()
    for x, y in zip(a, b[:3]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("kvd", ["bf16", "f32", "int8"])
def test_commit_path_bit_exact(kvd):
    ks = [16, 8, 5, 1, 12]
    w = _wk(f"commit-{kvd}", 8, 4, 128 if kvd != "f32" else 64, kvd, "bf16", ident=81)
    case = wl.make_case(w, device=DEV, ctx=[0, 15, 100, 7, 33], k=ks, with_logits=False)
    kv = paged_kv(case)
    batch = batch_of(case)
    parents = wl.make_tree(ks, device=DEV, seed=9)
    # accepted branches: root -> a chosen node (oracle walk of the parent array)
    par = np_(parents)
    cu = np_(case["cu_q"])
    n = np.zeros(len(ks), np.int32)
    path = -np.ones(sum(ks), np.int32)
    for b, k in enumerate(ks):
        if k == 0:
            continue
        j, chain = max(k - 1 - b % 2, 0), []
        while j >= 0:
            chain.append(j)
            p = int(par[cu[b] + j])
            j = p if 0 <= p < j else -1
        chain.reverse()
        n[b] = len(chain)
        path[cu[b]:cu[b] + len(chain)] = chain
    k0, v0 = np_(kv.k), np_(kv.v)
    s0 = (np_(kv.k_scale), np_(kv.v_scale)) if kvd == "int8" else None
    say(f"commit path {kvd}")
    tva.kv_commit_path(batch, torch.tensor(n, device=DEV), torch.tensor(path, device=DEV), kv)
    torch.cuda.synchronize()
    bt, ctx = np_(case["block_table"]), np_(case["ctx_lens"])
    if kvd == "int8":
        rk, rks = oracle.commit_path(k0, bt, ctx, cu, n, path, scale=s0[0])
        rv, rvs = oracle.commit_path(v0, bt, ctx, cu, n, path, scale=s0[1])
        assert np.array_equal(np_(kv.k_scale).view(np.uint16), rks.view(np.uint16))
        assert np.array_equal(np_(kv.v_scale).view(np.uint16), rvs.view(np.uint16))
    else:
        rk = oracle.commit_path(k0, bt, ctx, cu, n, path)
        rv = oracle.commit_path(v0, bt, ctx, cu, n, path)
    assert np.array_equal(np_(kv.k).view(np.uint8), rk.view(np.uint8))
    assert np.array_equal(np_(kv.v).view(np.uint8), rv.view(np.uint8))


def _two_caches(case, kvd):
    """Two independent copies of the case's cache in its stored format."""
    if kvd == "int8":
        kc, ks = tva.kv_quant_int8(case["k_pool"])
        vc, vs = tva.kv_quant_int8(case["v_pool"])
        mk = lambda: tva.PagedKV(kc.clone(), vc.clone(), case["block_table"], ks.clone(),
                                 vs.clone())
    else:
        dt = torch.float32 if kvd == "f32" else torch.bfloat16
        k, v = case["k_pool"].to(dt), case["v_pool"].to(dt)
        mk = lambda: tva.PagedKV(k.clone(), v.clone(), case["block_table"])
    return mk(), mk()


def _accept_commit_both_ways(case, parents, kvd):
    batch = batch_of(case)
    kv_a, kv_b = _two_caches(case, kvd)
    outs_a = tva.accept_tree(batch, case["logits"], case["draft_ids"], parents)
    tva.kv_commit_path(batch, outs_a[1], outs_a[3], kv_a)
    outs_b = tva.accept_tree_commit(batch, case["logits"], case["draft_ids"], parents, kv_b)
    torch.cuda.synchronize()
    for a, b in zip(outs_a, outs_b):
        assert torch.equal(a, b)
    for a, b in ((kv_a.k, kv_b.k), (kv_a.v, kv_b.v)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    if kvd == "int8":
        assert torch.equal(kv_a.k_scale.view(torch.int16), kv_b.k_scale.view(torch.int16))
        assert torch.equal(kv_a.v_scale.view(torch.int16), kv_b.v_scale.view(torch.int16))
    return outs_b


@pytest.mark.parametrize("kvd", ["bf16", "int8", "f32"])
def test_accept_tree_commit_equals_the_two_calls(kvd):
    """sva_accept_tree_commit gives the outputs of sva_accept_tree and the cache
    bytes of sva_kv_commit_path after it (ragged trees, empty and 16-node ones)."""
    ks = [16, 8, 5, 1, 0, 12]
    w = _wk(f"tc-{kvd}", 8, 4, 128 if kvd != "f32" else 64, kvd, "bf16", ident=86, vocab=4099,
            match=0.9)
    case = wl.make_case(w, device=DEV, ctx=[0, 15, 100, 7, 3, 33], k=ks, with_logits=False)
    parents = wl.make_tree(ks, device=DEV, seed=11)
    case.update(wl.make_tree_logits(w, ks, parents, device=DEV))
    say(f"accept_tree_commit {kvd}")
    outs = _accept_commit_both_ways(case, parents, kvd)
    assert int(outs[1].max()) > 1                      # some branch actually moves rows


def test_accept_tree_commit_full_size():
    """The token-tree benchmark shape (B=32, Hkv=8, d=128, V=128256)."""
    w = wl.WORKLOADS["tree8b"]
    case = wl.make_case(w, device=DEV, with_logits=False)
    parents = wl.make_tree(case["k_host"], device=DEV, seed=w.ident)
    case.update(wl.make_tree_logits(w, case["k_host"], parents, device=DEV))
    say("accept_tree_commit tree8b")
    _accept_commit_both_ways(case, parents, w.kv_dtype)


def test_tree_step_then_commit_matches_causal_after():
    """append -> tree attention -> accept -> commit; then the last accepted
    node's output equals causal attention over the committed cache."""
    ks = [8, 16, 4]
    w = _wk("step", 16, 4, 128, "bf16", "bf16", ident=82, vocab=3000, match=0.9)
    case = wl.make_case(w, device=DEV, ctx=[40, 120, 3], k=ks, with_logits=False)
    parents = wl.make_tree(ks, device=DEV, seed=2)
    case.update(wl.make_tree_logits(w, ks, parents, device=DEV))
    batch = batch_of(case)
    kv = paged_kv(case)
    tva.kv_append(batch, case["k_new"], case["v_new"], kv)
    masks = tva.tree_masks(batch, parents)
    out = tva.spec_verify_attn(batch, case["q"], kv, draft_mask=masks, out_dtype=torch.float32)
    ids, n, nxt, path = tva.accept_tree(batch, case["logits"], case["draft_ids"], parents)
    tva.kv_commit_path(batch, n, path, kv)
    torch.cuda.synchronize()
    nn, pp, cu = np_(n), np_(path), np_(case["cu_q"])
    # queries: the last accepted node's query placed at draft index n_b - 1
    qs, kk = [], []
    for b in range(len(ks)):
        m = int(nn[b])
        qb = torch.zeros(max(m, 1), w.Hq, w.d, dtype=case["q"].dtype, device=DEV)
        if m:
            qb[m - 1] = case["q"][cu[b] + int(pp[cu[b] + m - 1])]
        qs.append(qb)
        kk.append(max(m, 1))
    q2 = torch.cat(qs)
    cu2 = torch.tensor(np.concatenate([[0], np.cumsum(kk)]), dtype=torch.int32, device=DEV)
    b2 = tva.Batch(case["ctx_lens"], cu2)
    out2 = tva.spec_verify_attn(b2, q2, kv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(len(ks)):
        m = int(nn[b])
        if m == 0:
            continue
        node = cu[b] + int(pp[cu[b] + m - 1])
        got = out2[int(cu2[b]) + m - 1].float()
        want = out[node].float()
        assert (got - want).abs().max().item() <= 1e-2 * want.abs().max().item() + 1e-3


def test_tree8b_full_size_sampled():
    w = wl.WORKLOADS["tree8b"]
    say("tree8b full size")
    case = wl.make_case(w, device=DEV, with_logits=False)
    ks = case["k_host"]
    parents = wl.make_tree(ks, device=DEV, seed=w.ident)
    batch = batch_of(case)
    kv = paged_kv(case)
    masks = tva.tree_masks(batch, parents)
    out = tva.spec_verify_attn(batch, case["q"], kv, draft_mask=masks)
    torch.cuda.synchronize()
    pairs = [(0, 0), (7, 3), (19, 5), (31, 7)]
    om = _masks_oracle(case, parents)
    ref = oracle.spec_verify_attn(np_(case["q"]), np_(case["k_pool"]), np_(case["v_pool"]),
                                  np_(case["block_table"]), np_(case["ctx_lens"]),
                                  np_(case["cu_q"]), 1.0 / math.sqrt(w.d), select=pairs,
                                  draft_mask=om)
    assert_close(out, ref, "bf16", rows=rows_of_pairs(case, pairs))
