"""Pins for the attention oracle (CPU only).

Each pin comes from outside the oracle: a library routine (torch float64
scaled_dot_product_attention with an explicit bottom-right causal mask), a
pure-Python brute force on tiny shapes, closed forms, and invariants of the
definition in "Decoding Speculative Decoding from First Principles" (causal
verification of all drafts in one pass).
"""
import math

import numpy as np
import pytest
import torch

import oracle

PAGE = 16


def _paged_case(rng, B, Hq, Hkv, d, ctx, ks, extra_pages=2):
    """A random paged cache with a random physical page order."""
    npages = [-(-(c + k) // PAGE) for c, k in zip(ctx, ks)]
    P = sum(npages) + extra_pages
    perm = rng.permutation(P)
    maxp = max(npages + [1])
    bt = -np.ones((B, maxp), np.int64)
    off = 0
    for b in range(B):
        bt[b, : npages[b]] = perm[off: off + npages[b]]
        off += npages[b]
    T = sum(ks)
    q = rng.standard_normal((T, Hq, d)).astype(np.float32)
    kp = rng.standard_normal((P, Hkv, PAGE, d)).astype(np.float32)
    vp = rng.standard_normal((P, Hkv, PAGE, d)).astype(np.float32)
    cu = np.zeros(B + 1, np.int64)
    cu[1:] = np.cumsum(ks)
    return q, kp, vp, bt, np.array(ctx), cu


def _depage(pool, bt_row, n):
    """Independent gather for the pins: logical rows 0..n-1 of one sequence."""
    rows = []
    for p in range(n):
        rows.append(pool[bt_row[p // PAGE], :, p % PAGE, :])
    return np.stack(rows, 0) if rows else np.zeros((0,) + pool.shape[1:2] + pool.shape[3:])


SHAPES = [
    # B, Hq, Hkv, d, ctx, ks
    (1, 1, 1, 8, [0], [1]),
    (2, 4, 4, 16, [5, 17], [3, 1]),
    (3, 8, 2, 16, [40, 0, 16], [5, 2, 4]),
    (2, 6, 3, 32, [31, 33], [2, 6]),
    (3, 4, 1, 8, [15, 16, 1], [1, 0, 7]),
    # long speculated steps (step-level verification: tens to hundreds of drafts)
    (2, 7, 1, 16, [64, 3], [96, 40]),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_torch_sdpa_fp64(shape):
    B, Hq, Hkv, d, ctx, ks = shape
    rng = np.random.default_rng(11)
    q, kp, vp, bt, ctx_a, cu = _paged_case(rng, B, Hq, Hkv, d, ctx, ks)
    scale = 1.0 / math.sqrt(d)
    out = oracle.spec_verify_attn(q, kp, vp, bt, ctx_a, cu, scale)
    G = Hq // Hkv
    for b in range(B):
        k = ks[b]
        if k == 0:
            continue
        n = ctx[b] + k
        K = torch.from_numpy(_depage(kp, bt[b], n).astype(np.float64))   # [n, Hkv, d]
        V = torch.from_numpy(_depage(vp, bt[b], n).astype(np.float64))
        K = K.repeat_interleave(G, dim=1).permute(1, 0, 2)               # [Hq, n, d]
        V = V.repeat_interleave(G, dim=1).permute(1, 0, 2)
        Q = torch.from_numpy(q[cu[b]: cu[b + 1]].astype(np.float64)).permute(1, 0, 2)  # [Hq, k, d]
        # bottom-right aligned causal mask: query i sees keys 0 .. ctx+i
        mask = torch.arange(n)[None, :] <= (ctx[b] + torch.arange(k))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None], V[None], attn_mask=mask, scale=scale)[0]   # [Hq, k, d]
        got = torch.from_numpy(out[cu[b]: cu[b + 1]]).permute(1, 0, 2)
        assert torch.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_brute_force_pure_python():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, d, ctx, ks = 2, 4, 2, 4, [3, 18], [2, 3]
    q, kp, vp, bt, ctx_a, cu = _paged_case(rng, B, Hq, Hkv, d, ctx, ks)
    scale = 0.37
    out = oracle.spec_verify_attn(q, kp, vp, bt, ctx_a, cu, scale)
    G = Hq // Hkv
    for b in range(B):
        for i in range(ks[b]):
            for h in range(Hq):
                g = h // G
                keys = range(ctx[b] + i + 1)
                sc = []
                for p in keys:
                    pg, sl = bt[b][p // PAGE], p % PAGE
                    sc.append(scale * sum(float(q[cu[b] + i, h, c]) * float(kp[pg, g, sl, c])
                                          for c in range(d)))
                mx = max(sc)
                ex = [math.exp(s - mx) for s in sc]
                tot = sum(ex)
                for c in range(d):
                    acc = 0.0
                    for p, e in zip(keys, ex):
                        acc += e / tot * float(vp[bt[b][p // PAGE], g, p % PAGE, c])
                    assert abs(acc - out[cu[b] + i, h, c]) < 1e-12


def test_constant_value_rows_give_that_row():
    rng = np.random.default_rng(6)
    q, kp, vp, bt, ctx, cu = _paged_case(rng, 2, 4, 2, 16, [20, 7], [3, 4])
    row = rng.standard_normal(16)
    vp[:] = row.astype(np.float32)
    out = oracle.spec_verify_attn(q, kp, vp, bt, ctx, cu, 0.25)
    assert np.allclose(out, row.astype(np.float32).astype(np.float64)[None, None, :], rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(7)
    ctx, ks = [9, 30], [2, 3]
    q, kp, vp, bt, ctx_a, cu = _paged_case(rng, 2, 2, 1, 8, ctx, ks)
    kp[:] = kp[0, 0, 0]
    out = oracle.spec_verify_attn(q, kp, vp, bt, ctx_a, cu, 1.0)
    for b in range(2):
        Vb = _depage(vp, bt[b], ctx[b] + ks[b]).astype(np.float64)[:, 0, :]
        for i in range(ks[b]):
            mean = Vb[: ctx[b] + i + 1].mean(axis=0)
            for h in range(2):
                assert np.allclose(out[cu[b] + i, h], mean, atol=1e-13)


def test_single_draft_is_plain_decode_attention():
    rng = np.random.default_rng(8)
    ctx = [37]
    q, kp, vp, bt, ctx_a, cu = _paged_case(rng, 1, 2, 2, 8, ctx, [1])
    out = oracle.spec_verify_attn(q, kp, vp, bt, ctx_a, cu, 0.5)
    K = _depage(kp, bt[0], 38).astype(np.float64)
    V = _depage(vp, bt[0], 38).astype(np.float64)
    for h in range(2):
        s = 0.5 * K[:, h, :] @ q[0, h].astype(np.float64)      # every key, no mask
        w = np.exp(s - s.max())
        assert np.allclose(out[0, h], (w / w.sum()) @ V[:, h, :], atol=1e-13)


def test_weights_sum_to_one_and_cover_only_causal_keys():
    rng = np.random.default_rng(9)
    ctx, ks = [10, 0], [4, 3]
    q, kp, vp, bt, ctx_a, cu = _paged_case(rng, 2, 2, 2, 8, ctx, ks)
    _, w = oracle.spec_verify_attn(q, kp, vp, bt, ctx_a, cu, 0.3, return_weights=True)
    for (b, i, h), vec in w.items():
        assert len(vec) == ctx[b] + i + 1
        assert abs(vec.sum() - 1.0) < 1e-13
        assert (vec > 0).all()


def test_later_drafts_do_not_change_earlier_queries():
    rng = np.random.default_rng(10)
    ctx, ks = [21, 14], [5, 4]
    q, kp, vp, bt, ctx_a, cu = _paged_case(rng, 2, 4, 2, 16, ctx, ks)
    base = oracle.spec_verify_attn(q, kp, vp, bt, ctx_a, cu, 0.25)
    for b in range(2):
        for j in range(ks[b]):
            kp2, vp2 = kp.copy(), vp.copy()
            for jj in range(j + 1, ks[b]):
                p = ctx[b] + jj
                kp2[bt[b][p // PAGE], :, p % PAGE] += 100.0
                vp2[bt[b][p // PAGE], :, p % PAGE] = 1e6
            got = oracle.spec_verify_attn(q, kp2, vp2, bt, ctx_a, cu, 0.25)
            rows = slice(cu[b], cu[b] + j + 1)
            assert np.array_equal(got[rows], base[rows])


def test_page_permutation_invariance():
    rng = np.random.default_rng(12)
    q, kp, vp, bt, ctx, cu = _paged_case(rng, 3, 4, 2, 8, [16, 33, 5], [2, 3, 1])
    base = oracle.spec_verify_attn(q, kp, vp, bt, ctx, cu, 0.4)
    P = kp.shape[0]
    sigma = rng.permutation(P)                   # physical page p moves to sigma[p]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[sigma] = kp
    vp2[sigma] = vp
    bt2 = np.where(bt >= 0, sigma[np.maximum(bt, 0)], -1)
    got = oracle.spec_verify_attn(q, kp2, vp2, bt2, ctx, cu, 0.4)
    assert np.array_equal(got, base)


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(13)
    G = 3
    q, kp, vp, bt, ctx, cu = _paged_case(rng, 2, 6, 2, 8, [12, 19], [2, 2])
    gqa = oracle.spec_verify_attn(q, kp, vp, bt, ctx, cu, 0.3)
    mha = oracle.spec_verify_attn(q, np.repeat(kp, G, axis=1), np.repeat(vp, G, axis=1),
                                  bt, ctx, cu, 0.3)
    assert np.allclose(gqa, mha, rtol=0, atol=1e-14)


def test_query_scale_trade():
    rng = np.random.default_rng(14)
    q, kp, vp, bt, ctx, cu = _paged_case(rng, 1, 2, 2, 8, [25], [3])
    a = oracle.spec_verify_attn(q, kp, vp, bt, ctx, cu, 0.5)
    b = oracle.spec_verify_attn(q * np.float32(4.0), kp, vp, bt, ctx, cu, 0.125)
    assert np.allclose(a, b, atol=1e-13)


def test_int8_pool_is_dequantised_codes_times_scales():
    rng = np.random.default_rng(15)
    q, kp, vp, bt, ctx, cu = _paged_case(rng, 2, 4, 2, 16, [16, 3], [2, 4])
    P, Hkv = kp.shape[:2]
    kc, ks_ = oracle.kv_quant_int8(kp.reshape(-1, 16))
    vc, vs_ = oracle.kv_quant_int8(vp.reshape(-1, 16))
    kc, vc = kc.reshape(kp.shape), vc.reshape(vp.shape)
    ks_, vs_ = ks_.reshape(P, Hkv, PAGE), vs_.reshape(P, Hkv, PAGE)
    got = oracle.spec_verify_attn(q, kc, vc, bt, ctx, cu, 0.25, k_scale=ks_, v_scale=vs_)
    kd = kc.astype(np.float64) * ks_.astype(np.float64)[..., None]
    vd = vc.astype(np.float64) * vs_.astype(np.float64)[..., None]
    ref = oracle.spec_verify_attn(q, kd, vd, bt, ctx, cu, 0.25)
    assert np.array_equal(got, ref)
