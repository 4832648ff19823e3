"""Property-based pins of the oracle (CPU only, hypothesis): small random
shapes -- B <= 3 sequences, contexts S <= 40, k <= 5 drafts, d in {8, 64} --
each checked against something outside the oracle.

* attention: torch float64 scaled_dot_product_attention on the de-paged
  K/V with an explicit bottom-right causal mask ("Decoding Speculative
  Decoding from First Principles", section "Speculating to get sequence
  parallelism during decode": draft i sees the context and drafts 0 .. i);
  draft j's output unchanged when later drafts change;
* INT8 ("CXL-SpecKV", Algorithm 2, scaling and quantisation steps): the
  round-trip bound |x - c s| <= s / 2, the absmax element at +-127, odd
  symmetry, idempotence on dequantised rows;
* acceptance (same blog section): the longest prefix equal to numpy's row
  argmax, 0 <= n <= k, and the bonus token when all drafts match;
* page lists ("HeteroReason", KV Cache Management Unit): every page in exactly
  one place after allocation and reclamation.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

PAGE = 16
SETTINGS = settings(max_examples=40, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def batches(draw):
    B = draw(st.integers(1, 3))
    Hkv = draw(st.sampled_from([1, 2]))
    G = draw(st.sampled_from([1, 2, 3]))
    d = draw(st.sampled_from([8, 64]))
    ctx = draw(st.lists(st.integers(0, 40), min_size=B, max_size=B))
    ks = draw(st.lists(st.integers(0, 5), min_size=B, max_size=B))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return B, Hkv * G, Hkv, d, ctx, ks, seed


def _paged(B, Hq, Hkv, d, ctx, ks, seed):
    rng = np.random.default_rng(seed)
    npages = [-(-(c + k) // PAGE) for c, k in zip(ctx, ks)]
    P = sum(npages) + 1
    perm = rng.permutation(P)
    bt = -np.ones((B, max(npages + [1])), np.int64)
    off = 0
    for b in range(B):
        bt[b, :npages[b]] = perm[off:off + npages[b]]
        off += npages[b]
    q = rng.standard_normal((sum(ks), Hq, d)).astype(np.float32)
    kp = rng.standard_normal((P, Hkv, PAGE, d)).astype(np.float32)
    vp = rng.standard_normal((P, Hkv, PAGE, d)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(ks)]).astype(np.int64)
    return q, kp, vp, bt, np.array(ctx), cu


def _rows(pool, bt_row, n):
    return np.stack([pool[bt_row[p // PAGE], :, p % PAGE, :] for p in range(n)], 0)


@SETTINGS
@given(batches())
def test_attention_equals_masked_sdpa(case):
    B, Hq, Hkv, d, ctx, ks, seed = case
    q, kp, vp, bt, ctx_a, cu = _paged(B, Hq, Hkv, d, ctx, ks, seed)
    scale = 1.0 / math.sqrt(d)
    out = oracle.spec_verify_attn(q, kp, vp, bt, ctx_a, cu, scale)
    G = Hq // Hkv
    for b in range(B):
        k, n = ks[b], ctx[b] + ks[b]
        if k == 0:
            continue
        K = torch.from_numpy(_rows(kp, bt[b], n).astype(np.float64))
        V = torch.from_numpy(_rows(vp, bt[b], n).astype(np.float64))
        K = K.repeat_interleave(G, dim=1).permute(1, 0, 2)
        V = V.repeat_interleave(G, dim=1).permute(1, 0, 2)
        Q = torch.from_numpy(q[cu[b]:cu[b + 1]].astype(np.float64)).permute(1, 0, 2)
        mask = torch.arange(n)[None, :] <= (ctx[b] + torch.arange(k))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None], V[None], attn_mask=mask, scale=scale)[0]
        got = torch.from_numpy(out[cu[b]:cu[b + 1]]).permute(1, 0, 2)
        assert torch.allclose(got, ref, rtol=1e-11, atol=1e-11)


@SETTINGS
@given(batches(), st.integers(0, 4))
def test_attention_prefix_invariance(case, j):
    """Draft j's output does not depend on the K/V rows of later drafts."""
    B, Hq, Hkv, d, ctx, ks, seed = case
    q, kp, vp, bt, ctx_a, cu = _paged(B, Hq, Hkv, d, ctx, ks, seed)
    base = oracle.spec_verify_attn(q, kp, vp, bt, ctx_a, cu, 0.3)
    kp2, vp2 = kp.copy(), vp.copy()
    for b in range(B):
        for i in range(j + 1, ks[b]):
            pos = ctx[b] + i
            kp2[bt[b][pos // PAGE], :, pos % PAGE] += 5.0
            vp2[bt[b][pos // PAGE], :, pos % PAGE] -= 7.0
    pert = oracle.spec_verify_attn(q, kp2, vp2, bt, ctx_a, cu, 0.3)
    for b in range(B):
        rows = slice(cu[b], cu[b] + min(j + 1, ks[b]))
        assert np.array_equal(base[rows], pert[rows])


@SETTINGS
@given(st.integers(0, 2 ** 31 - 1), st.sampled_from([8, 64]), st.floats(1e-3, 1e3))
def test_int8_round_trip_properties(seed, d, mag):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((6, d)) * mag).astype(np.float32)
    codes, s16 = oracle.kv_quant_int8(x)
    s = s16.astype(np.float64)
    deq = codes.astype(np.float64) * s[:, None]
    assert (np.abs(x - deq) <= s[:, None] / 2 * (1 + 1e-12)).all()       # round-trip bound
    amax = np.abs(x).argmax(axis=1)
    assert (np.abs(codes[np.arange(6), amax]) == 127).all()                # absmax at +-127
    assert (np.abs(codes) <= 127).all()
    neg_codes, neg_s = oracle.kv_quant_int8(-x)                           # odd symmetry
    assert np.array_equal(neg_codes, -codes) and np.array_equal(neg_s, s16)
    again, s_again = oracle.kv_quant_int8(deq.astype(np.float32))          # idempotence
    assert np.array_equal(again, codes) and np.array_equal(s_again, s16)


@SETTINGS
@given(st.lists(st.integers(0, 5), min_size=1, max_size=3), st.integers(0, 2 ** 31 - 1),
       st.floats(0.0, 1.0))
def test_acceptance_is_the_longest_prefix_of_argmax_matches(ks, seed, p_match):
    rng = np.random.default_rng(seed)
    V = 50
    B = len(ks)
    cu = np.concatenate([[0], np.cumsum(ks)])
    logits = rng.standard_normal((sum(ks) + B, V)).astype(np.float32)
    t = logits.argmax(axis=1)
    drafts = []
    for b, k in enumerate(ks):
        for j in range(k):
            tj = int(t[cu[b] + b + j])
            drafts.append(tj if rng.random() < p_match else (tj + 1) % V)
    drafts = np.array(drafts, np.int64)
    ids, n, nxt = oracle.accept_prefix(logits, drafts, cu)
    assert np.array_equal(ids, t)
    for b, k in enumerate(ks):
        row0 = cu[b] + b
        want = 0
        while want < k and drafts[cu[b] + want] == t[row0 + want]:
            want += 1
        assert n[b] == want and 0 <= n[b] <= k
        assert nxt[b] == t[row0 + want]                  # the n+1-th emitted token


@SETTINGS
@given(st.integers(0, 2 ** 31 - 1), st.integers(1, 5), st.integers(1, 12))
def test_page_lists_conserve_pages(seed, B, max_pages):
    rng = np.random.default_rng(seed)
    P = B * max_pages + 5
    perm = rng.permutation(P)
    bt = -np.ones((B, max_pages), np.int64)
    used = 0
    for b in range(B):
        n = int(rng.integers(0, max_pages + 1))
        bt[b, :n] = perm[used:used + n]
        used += n
    fl = np.concatenate([perm[used:], -np.ones(used + 8, np.int64)])    # room for every page
    count = P - used
    for _ in range(5):
        lens = rng.integers(0, PAGE * max_pages - 8, B)
        ks = rng.integers(0, 9, B)
        cu = np.concatenate([[0], np.cumsum(ks)])
        bt, count = oracle.alloc_pages(bt, lens, cu, fl, count)
        lens = lens + rng.integers(0, ks + 1)
        bt, fl, count = oracle.reclaim_pages(bt, lens, fl, count)
        assigned = bt[bt >= 0].tolist()
        assert sorted(assigned + fl[:count].tolist()) == list(range(P))
        for b in range(B):
            for j in range(max_pages):
                if bt[b, j] >= 0:
                    assert PAGE * j < lens[b]
