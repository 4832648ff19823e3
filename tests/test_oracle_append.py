"""Pins for the append oracle and the multi-step commit / rollback loop (CPU).

"HeteroReason", workflow Phase 3 and the KVMU modes (Fig. 7): accepted rows
stay valid, the rows of rejected drafts become invalid when the valid pointer
does not move past them.  Here commit is S_b <- S_b + n_b and the next step's
drafts overwrite the invalid rows.
"""
import math

import numpy as np

import oracle

PAGE = 16


def _layout(rng, ctx, ks, extra=0, slack=0):
    npages = [-(-(c + k + slack) // PAGE) for c, k in zip(ctx, ks)]
    P = sum(npages) + extra
    perm = rng.permutation(P)
    bt = -np.ones((len(ctx), max(npages)), np.int64)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[off: off + n]
        off += n
    return P, bt


def test_rows_land_at_their_logical_positions():
    rng = np.random.default_rng(2)
    ctx, ks, Hkv, d = [15, 0, 33], [3, 2, 1], 2, 8
    P, bt = _layout(rng, ctx, ks)
    kp = np.zeros((P, Hkv, PAGE, d)); vp = np.zeros((P, Hkv, PAGE, d))
    T = sum(ks)
    kn = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(ks)])
    k2, v2, _, _ = oracle.kv_append(kn, vn, kp, vp, bt, np.array(ctx), cu, "f32")
    written = np.zeros((P, Hkv, PAGE), bool)
    for b in range(3):
        for i in range(ks[b]):
            p = ctx[b] + i
            pg, sl = bt[b][p // PAGE], p % PAGE
            assert np.array_equal(k2[pg, :, sl], kn[cu[b] + i])
            assert np.array_equal(v2[pg, :, sl], vn[cu[b] + i])
            written[pg, :, sl] = True
    assert (k2[~written] == 0).all() and (v2[~written] == 0).all()


def test_int8_and_bf16_caches_store_the_rounded_row():
    rng = np.random.default_rng(3)
    ctx, ks, Hkv, d = [5, 20], [2, 3], 2, 16
    P, bt = _layout(rng, ctx, ks)
    T = sum(ks)
    cu = np.concatenate([[0], np.cumsum(ks)])
    kn = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    zc = np.zeros((P, Hkv, PAGE, d), np.int8)
    zs = np.zeros((P, Hkv, PAGE), np.float16)
    kc, vc, ksc, vsc = oracle.kv_append(kn, vn, zc, zc, bt, np.array(ctx), cu, "int8", zs, zs)
    kb, vb, _, _ = oracle.kv_append(kn, vn, np.zeros((P, Hkv, PAGE, d)), np.zeros((P, Hkv, PAGE, d)),
                                    bt, np.array(ctx), cu, "bf16")
    for b in range(2):
        for i in range(ks[b]):
            p = ctx[b] + i
            pg, sl = bt[b][p // PAGE], p % PAGE
            c, s = oracle.kv_quant_int8(kn[cu[b] + i])
            assert np.array_equal(kc[pg, :, sl], c) and np.array_equal(ksc[pg, :, sl], s)
            assert np.array_equal(kb[pg, :, sl], oracle.round_to_bf16(kn[cu[b] + i]))


def test_draft_verify_commit_loop_never_reads_rejected_rows():
    """Three verification steps on the oracle.  After each step the rows of the
    rejected drafts are poisoned with NaN; the commit moves S_b by the accepted
    count only, so the next step must never see a NaN."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, d, V, steps, kmax = 3, 4, 2, 8, 11, 3, 4
    ctx = [7, 16, 30]
    P, bt = _layout(rng, ctx, [kmax] * B, slack=steps * kmax)
    kp = rng.standard_normal((P, Hkv, PAGE, d))
    vp = rng.standard_normal((P, Hkv, PAGE, d))
    for step in range(steps):
        ks = [int(v) for v in rng.integers(1, kmax + 1, B)]
        cu = np.concatenate([[0], np.cumsum(ks)])
        T = cu[-1]
        kn = rng.standard_normal((T, Hkv, d)).astype(np.float32)
        vn = rng.standard_normal((T, Hkv, d)).astype(np.float32)
        kp, vp, _, _ = oracle.kv_append(kn, vn, kp, vp, bt, np.array(ctx), cu, "f32")
        q = rng.standard_normal((T, Hq, d)).astype(np.float32)
        out = oracle.spec_verify_attn(q, kp, vp, bt, np.array(ctx), cu, 1 / math.sqrt(d))
        assert np.isfinite(out).all()
        logits = rng.standard_normal((T + B, V)).astype(np.float32)
        t = oracle.argmax_rows(logits)
        drafts = np.array([t[cu[b] + b + j] if rng.random() < 0.6 else (t[cu[b] + b + j] + 1) % V
                           for b in range(B) for j in range(ks[b])])
        _, n, _ = oracle.accept_prefix(logits, drafts, cu)
        for b in range(B):
            for j in range(n[b], ks[b]):                     # rejected rows: invalid
                p = ctx[b] + j
                kp[bt[b][p // PAGE], :, p % PAGE] = np.nan
                vp[bt[b][p // PAGE], :, p % PAGE] = np.nan
            ctx[b] += int(n[b])                               # commit
