"""GPU parity of sva_kvmu_apply against the KVMU oracle (through the C ABI):
random per-sequence mode sequences applied step by step (bit-exact pointer
triplets and ctx_lens), the uniform-mode form, and a three-step verification
loop whose committed lengths stay on the device: append -> attention ->
greedy acceptance -> Prefix commit, checked against the oracle's acceptance
and attention on the same inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import token_verify_attention_amd as tva
from oracle.kvmu import kvmu_apply as kvmu_ref
from token_verify_attention_amd import workloads as wl
from gpu_helpers import assert_close, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_random_mode_sequences_bit_exact():
    rng = np.random.default_rng(4)
    B = 300
    st_h = np.zeros((B, 3), np.int64)
    st = torch.zeros(B, 3, dtype=torch.int32, device=DEV)
    lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    say("kvmu random sequences")
    for step in range(60):
        mode = rng.integers(0, 6, B).astype(np.int32)          # 5 = unknown: no change
        arg = rng.integers(-3, 40, B).astype(np.int32)
        if step == 0:
            mode[:] = 0
            arg = rng.integers(0, 5000, B).astype(np.int32)
        tva.kvmu_apply(st, torch.tensor(mode, device=DEV), torch.tensor(arg, device=DEV), lens)
        known = mode < 5
        nxt = kvmu_ref(st_h, np.where(known, mode, 0), arg)
        st_h = np.where(known[:, None], nxt, st_h)
    torch.cuda.synchronize()
    assert np.array_equal(np_(st).astype(np.int64), st_h)
    assert np.array_equal(np_(lens).astype(np.int64), st_h[:, 0])


def test_uniform_modes():
    B = 5
    st = torch.tensor([[10, 12, 20]] * B, dtype=torch.int32, device=DEV)
    arg = torch.tensor([0, 1, 2, 3, 30], dtype=torch.int32, device=DEV)
    tva.kvmu_apply(st, tva.KVMU_PREFIX, arg)
    torch.cuda.synchronize()
    want = kvmu_ref(np.array([[10, 12, 20]] * B), [4] * B, np_(arg))
    assert np.array_equal(np_(st).astype(np.int64), want)
    tva.kvmu_apply(st, tva.KVMU_SPECULATE, arg)
    tva.kvmu_apply(st, tva.KVMU_ACCEPT)
    torch.cuda.synchronize()
    want = kvmu_ref(kvmu_ref(want, [1] * B, np_(arg)), [2] * B, [0] * B)
    assert np.array_equal(np_(st).astype(np.int64), want)


def test_verification_loop_commits_on_device():
    w = wl.Workload("loop", 1, 16, 4, 128, 0, 1, "bf16", "bf16", 1.0, 3000, 0.7, True, 97)
    ks = [4, 8, 1, 6]
    ctx0 = [30, 200, 0, 77]
    steps = 3
    B = len(ks)
    # a cache with room for every step's drafts
    case = wl.make_case(w, device=DEV, ctx=[c + steps * max(ks) for c in ctx0], k=ks)
    bt = case["block_table"]
    kv = tva.PagedKV(case["k_pool"], case["v_pool"], bt)
    state = torch.tensor([[c, c, c] for c in ctx0], dtype=torch.int32, device=DEV)
    ctx = torch.tensor(ctx0, dtype=torch.int32, device=DEV)
    cu = case["cu_q"]
    host_len = list(ctx0)
    max_len = max(ctx0) + steps * max(ks) + max(ks)
    for s in range(steps):
        say(f"kvmu loop step {s}")
        step = wl.make_case(w, device=DEV, ctx=host_len, k=ks, seed_offset=s + 1)
        batch = tva.Batch(ctx, cu, total_q=sum(ks), max_q=max(ks), max_len=max_len)
        tva.kvmu_apply(state, tva.KVMU_SPECULATE, torch.tensor(ks, dtype=torch.int32, device=DEV))
        tva.kv_append(batch, step["k_new"], step["v_new"], kv)
        out = tva.spec_verify_attn(batch, step["q"], kv, out_dtype=torch.float32)
        ids, n, nxt = tva.accept_prefix(batch, step["logits"], step["draft_ids"])
        tva.kvmu_apply(state, tva.KVMU_PREFIX, n, ctx_lens=ctx)
        torch.cuda.synchronize()
        # oracle on the same inputs: attention over the cache as it is now
        ref = oracle.spec_verify_attn(np_(step["q"]), np_(kv.k), np_(kv.v), np_(bt),
                                      np.array(host_len), np_(cu), 1.0 / math.sqrt(w.d))
        assert_close(out, ref, "bf16")
        _, rn, _ = oracle.accept_prefix(np_(step["logits"]), np_(step["draft_ids"]), np_(cu))
        assert np.array_equal(np_(n), rn)
        host_len = [h + int(x) for h, x in zip(host_len, rn)]
        assert np_(ctx).tolist() == host_len
        assert np_(state).tolist() == [[h, h, h] for h in host_len]


def _random_tables(rng, B, max_pages, P):
    """A block table whose sequences hold random numbers of pages (a random
    permutation of 0 .. P-1 spread over them, some entries left -1) and the
    pages it does not use as a free list."""
    perm = rng.permutation(P)
    bt = np.full((B, max_pages), -1, np.int64)
    used = 0
    for b in range(B):
        n = int(rng.integers(0, max_pages + 1))
        n = min(n, P - used)
        bt[b, :n] = perm[used:used + n]
        if n > 2 and rng.random() < 0.3:
            bt[b, int(rng.integers(0, n))] = -1          # a hole
        used += n
    return bt, perm[used:]


@pytest.mark.parametrize("B,max_pages", [(7, 30), (300, 700), (2, 4000)])
def test_reclaim_and_alloc_bit_exact(B, max_pages):
    rng = np.random.default_rng(B + max_pages)
    P = B * max_pages // 2 + 10
    bt_h, free = _random_tables(rng, B, max_pages, P)
    cap = P + 64
    fl_h = np.full(cap, -1, np.int64)
    fl_h[:len(free)] = free
    count_h = len(free)
    bt = torch.tensor(bt_h, dtype=torch.int32, device=DEV)
    fl = torch.tensor(fl_h, dtype=torch.int32, device=DEV)
    cnt = torch.tensor([count_h], dtype=torch.int32, device=DEV)
    say(f"pages B={B} max_pages={max_pages}")
    for it in range(4):
        lens_h = rng.integers(-5, 16 * max_pages + 40, B)
        ks_h = rng.integers(0, 17, B)
        cu_h = np.concatenate([[0], np.cumsum(ks_h)])
        lens = torch.tensor(lens_h, dtype=torch.int32, device=DEV)
        cu = torch.tensor(cu_h, dtype=torch.int32, device=DEV)
        tva.kv_reclaim_pages(lens, bt, fl, cnt)
        bt_h, fl_h, count_h = oracle.reclaim_pages(bt_h, lens_h, fl_h, count_h)
        torch.cuda.synchronize()
        assert np.array_equal(np_(bt).astype(np.int64), bt_h), it
        assert int(cnt.item()) == count_h
        assert np.array_equal(np_(fl).astype(np.int64)[:min(count_h, cap)],
                              fl_h[:min(count_h, cap)])
        # the next step's rows take pages back (lengths before its drafts)
        lens_h = np.maximum(lens_h - rng.integers(0, 50, B), 0)
        lens = torch.tensor(lens_h, dtype=torch.int32, device=DEV)
        batch = tva.Batch(lens, cu, total_q=int(cu_h[-1]), max_q=16,
                          max_len=int((lens_h + ks_h).max()))
        tva.kv_alloc_pages(batch, bt, fl, cnt)
        bt_h, count_h = oracle.alloc_pages(bt_h, lens_h, cu_h, fl_h, count_h)
        torch.cuda.synchronize()
        assert np.array_equal(np_(bt).astype(np.int64), bt_h), it
        assert int(cnt.item()) == count_h


def test_reclaim_into_a_full_list_counts_past_its_capacity():
    bt_h = np.array([[3, 4, 5, 6], [7, 8, -1, -1]])
    fl = torch.tensor([1, 2], dtype=torch.int32, device=DEV)          # capacity 2, full
    cnt = torch.tensor([2], dtype=torch.int32, device=DEV)
    bt = torch.tensor(bt_h, dtype=torch.int32, device=DEV)
    tva.kv_reclaim_pages(torch.tensor([16, 0], dtype=torch.int32, device=DEV), bt, fl, cnt)
    torch.cuda.synchronize()
    assert np_(bt).tolist() == [[3, -1, -1, -1], [-1, -1, -1, -1]]
    assert int(cnt.item()) == 7 and np_(fl).tolist() == [1, 2]


def test_graph_captured_verification_loop():
    """One verification step -- Speculation, page allocation, append and
    verification (one call), greedy acceptance, Prefix commit into ctx_lens,
    page reclamation -- captured once in a HIP graph and replayed for three
    steps, the inputs of each step copied into the captured buffers between
    replays.  Every replay is checked against the oracle's step on the same
    inputs: attention within the bar; acceptance, lengths, pointer triplets,
    block table, free list and every cache byte bit-exact."""
    w = wl.Workload("graph-loop", 1, 16, 4, 128, 0, 1, "bf16", "bf16", 1.0, 3000, 0.7, True, 98)
    ks = [4, 8, 1, 6]
    ctx0 = [30, 200, 0, 77]
    steps, B = 3, len(ks)
    T = sum(ks)
    scale = 1.0 / math.sqrt(w.d)
    # pool: the case's pages, of which only the contexts' stay assigned
    base = wl.make_case(w, device=DEV, ctx=[c + 40 for c in ctx0], k=ks, extra_pages=16)
    bt_full = np_(base["block_table"]).astype(np.int64)
    P = int(base["k_pool"].shape[0])
    bt_h = np.full_like(bt_full, -1)
    for b, c in enumerate(ctx0):
        n = -(-c // 16)
        bt_h[b, :n] = bt_full[b, :n]
    free = sorted(set(range(P)) - set(bt_h[bt_h >= 0].tolist()))
    fl_h = np.array(free, np.int64)
    count_h = len(free)
    kp_h, vp_h = np_(base["k_pool"]), np_(base["v_pool"])
    bt = torch.tensor(bt_h, dtype=torch.int32, device=DEV)
    fl = torch.tensor(fl_h, dtype=torch.int32, device=DEV)
    cnt = torch.tensor([count_h], dtype=torch.int32, device=DEV)
    kv = tva.PagedKV(base["k_pool"], base["v_pool"], bt)
    ctx = torch.tensor(ctx0, dtype=torch.int32, device=DEV)
    state = torch.tensor([[c, c, c] for c in ctx0], dtype=torch.int32, device=DEV)
    k_t = torch.tensor(ks, dtype=torch.int32, device=DEV)
    batch = tva.Batch(ctx, base["cu_q"], total_q=T, max_q=max(ks),
                      max_len=max(ctx0) + (steps + 1) * max(ks))
    cu_h = np_(base["cu_q"])
    # the captured buffers
    q_buf = torch.empty_like(base["q"])
    kn_buf, vn_buf = torch.empty_like(base["k_new"]), torch.empty_like(base["v_new"])
    lg_buf = torch.empty_like(base["logits"])
    dr_buf = torch.empty_like(base["draft_ids"])
    out = torch.empty(q_buf.shape, dtype=torch.float32, device=DEV)
    ids = torch.empty(T + B, dtype=torch.int32, device=DEV)
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    nxt = torch.empty(B, dtype=torch.int32, device=DEV)
    verify = tva.prepare_spec_verify_attn_append(batch, q_buf, kv, kn_buf, vn_buf, out)
    accept = tva.prepare_accept_prefix(batch, lg_buf, dr_buf, ids, n, nxt)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    say("graph loop: capture")
    with torch.cuda.graph(g):
        tva.kvmu_apply(state, tva.KVMU_SPECULATE, k_t)
        tva.kv_alloc_pages(batch, bt, fl, cnt)
        verify()
        accept()
        tva.kvmu_apply(state, tva.KVMU_PREFIX, n, ctx_lens=ctx)
        tva.kv_reclaim_pages(ctx, bt, fl, cnt)
    torch.cuda.synchronize()
    len_h = np.array(ctx0, np.int64)
    for s in range(steps):
        say(f"graph loop: replay {s}")
        step = wl.make_case(w, device=DEV, ctx=len_h.tolist(), k=ks, seed_offset=s + 1)
        for dst, src in ((q_buf, "q"), (kn_buf, "k_new"), (vn_buf, "v_new"),
                         (lg_buf, "logits"), (dr_buf, "draft_ids")):
            dst.copy_(step[src])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # the oracle's step on the same inputs
        bt_h, count_h = oracle.alloc_pages(bt_h, len_h, cu_h, fl_h, count_h)
        kp_h, vp_h, _, _ = oracle.kv_append(np_(step["k_new"]), np_(step["v_new"]), kp_h, vp_h,
                                            bt_h, len_h, cu_h, "bf16")
        ref = oracle.spec_verify_attn(np_(step["q"]), kp_h, vp_h, bt_h, len_h, cu_h, scale)
        rt, rn, rx = oracle.accept_prefix(np_(step["logits"]), np_(step["draft_ids"]), cu_h)
        len_h = len_h + rn
        bt_h, fl_h, count_h = oracle.reclaim_pages(bt_h, len_h, fl_h, count_h)
        assert_close(out, ref, "bf16")
        assert np.array_equal(np_(ids), rt) and np.array_equal(np_(n), rn)
        assert np.array_equal(np_(nxt), rx)
        assert np_(ctx).tolist() == len_h.tolist()
        assert np_(state).tolist() == [[h, h, h] for h in len_h.tolist()]
        assert np.array_equal(np_(bt).astype(np.int64), bt_h)
        assert int(cnt.item()) == count_h
        assert np.array_equal(np_(fl).astype(np.int64)[:count_h], fl_h[:count_h])
        assert np.array_equal(np_(kv.k), kp_h) and np.array_equal(np_(kv.v), vp_h)
        assert (rn < np.array(ks)).any() or s > 0     # some rejection happens
