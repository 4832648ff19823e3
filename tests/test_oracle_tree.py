"""Pins for the tree-verification oracle (CPU only).

"Decoding Speculative Decoding from First Principles", section "Tree based
verification": tree attention relates each draft to its lineage only, and the
accepted continuation is the longest branch the target agrees with.  Each pin
reaches the oracle's result by another route: a boolean transitive closure
for the ancestor masks, torch's float64 scaled_dot_product_attention with the
tree mask, brute-force enumeration of root-to-node paths, chain trees that
reduce to the (separately pinned) causal functions, and the invariant that
committing the accepted branch turns tree attention into causal attention.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle

PAGE = 16


def random_parents(rng, k, p_chain=0.5):
    """Topological parent array: mostly extend the previous node, else branch."""
    par = []
    for i in range(k):
        if i > 0 and rng.random() < p_chain:
            par.append(i - 1)
        else:
            par.append(int(rng.integers(-1, i)))      # -1 .. i-1
    return par


def closure_masks(parents):
    """Visibility by boolean transitive closure: reach[i, j] = j is i or an ancestor."""
    k = len(parents)
    adj = np.zeros((k, k), dtype=bool)
    for i, p in enumerate(parents):
        if p >= 0:
            adj[i, p] = True
    reach = np.eye(k, dtype=bool) | adj
    for _ in range(k):
        reach = reach | (reach.astype(np.int64) @ reach.astype(np.int64) > 0)
    return [int(sum(1 << j for j in range(k) if reach[i, j])) for i in range(k)], reach


def test_masks_match_transitive_closure():
    rng = np.random.default_rng(11)
    for trial in range(50):
        ks = [int(rng.integers(0, 17)) for _ in range(3)]
        cu = np.concatenate([[0], np.cumsum(ks)])
        parents, want = [], []
        for k in ks:
            par = random_parents(rng, k)
            parents += par
            want += closure_masks(par)[0]
        got = oracle.ancestor_masks(np.array(parents, dtype=np.int64), cu)
        assert list(got) == want


def test_masks_special_trees():
    cu = np.array([0, 6, 11])
    chain = [-1, 0, 1, 2, 3, 4] + [-1, 0, 1, 2, 3]
    assert list(oracle.ancestor_masks(chain, cu)) == [(1 << (i + 1)) - 1 for i in range(6)] + \
        [(1 << (i + 1)) - 1 for i in range(5)]
    star = [-1] * 11
    assert list(oracle.ancestor_masks(star, cu)) == [1 << i for i in range(6)] + [1 << i for i in range(5)]
    # out-of-range parents (self, later node, < -1) are read as roots
    bad = [-1, 1, 5, -7, 2, 0]
    assert list(oracle.ancestor_masks(bad, [0, 6])) == [1, 2, 4, 8, 20, 33]


def _paged(rng, B, Hq, Hkv, d, ctx, ks):
    npages = [-(-(c + k) // PAGE) for c, k in zip(ctx, ks)]
    P = sum(npages) + 1
    perm = rng.permutation(P)
    bt = -np.ones((B, max(npages + [1])), np.int64)
    off = 0
    for b in range(B):
        bt[b, : npages[b]] = perm[off: off + npages[b]]
        off += npages[b]
    T = sum(ks)
    q = rng.standard_normal((T, Hq, d))
    kp = rng.standard_normal((P, Hkv, PAGE, d))
    vp = rng.standard_normal((P, Hkv, PAGE, d))
    cu = np.concatenate([[0], np.cumsum(ks)]).astype(np.int64)
    return q, kp, vp, bt, np.array(ctx), cu


def test_chain_mask_equals_causal():
    rng = np.random.default_rng(3)
    ctx, ks = [20, 0, 33], [5, 3, 7]
    q, kp, vp, bt, c, cu = _paged(rng, 3, 8, 2, 16, ctx, ks)
    chain = oracle.ancestor_masks(np.concatenate([[-1] + list(range(k - 1)) for k in ks]), cu)
    a = oracle.spec_verify_attn(q, kp, vp, bt, c, cu, 0.25)
    b = oracle.spec_verify_attn(q, kp, vp, bt, c, cu, 0.25, draft_mask=chain)
    np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_tree_attention_matches_torch_sdpa(seed):
    rng = np.random.default_rng(100 + seed)
    B, Hq, Hkv, d = 2, 6, 3, 16
    ctx = [int(rng.integers(0, 40)) for _ in range(B)]
    ks = [int(rng.integers(1, 12)) for _ in range(B)]
    q, kp, vp, bt, c, cu = _paged(rng, B, Hq, Hkv, d, ctx, ks)
    parents, masks, reaches = [], [], []
    for k in ks:
        par = random_parents(rng, k)
        parents += par
        m, reach = closure_masks(par)
        masks += m
        reaches.append(reach)
    scale = 1.0 / math.sqrt(d)
    got = oracle.spec_verify_attn(q, kp, vp, bt, c, cu, scale, draft_mask=np.array(masks))
    G = Hq // Hkv
    for b in range(B):
        S, k, q0 = ctx[b], ks[b], int(cu[b])
        n = S + k
        K = np.stack([kp[bt[b][p // PAGE], :, p % PAGE, :] for p in range(n)])  # [n, Hkv, d]
        V = np.stack([vp[bt[b][p // PAGE], :, p % PAGE, :] for p in range(n)])
        allow = np.zeros((k, n), dtype=bool)
        allow[:, :S] = True
        allow[:, S:] = reaches[b]
        Kt = torch.tensor(np.repeat(K, G, axis=1)).permute(1, 0, 2)    # [Hq, n, d]
        Vt = torch.tensor(np.repeat(V, G, axis=1)).permute(1, 0, 2)
        Qt = torch.tensor(q[q0:q0 + k]).permute(1, 0, 2)               # [Hq, k, d]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Qt, Kt, Vt, attn_mask=torch.tensor(allow), scale=scale).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(got[q0:q0 + k], ref, rtol=1e-11, atol=1e-12)


def test_star_tree_is_context_plus_self():
    """Each root-level draft sees the context and its own row only."""
    rng = np.random.default_rng(9)
    S, k, d = 21, 6, 8
    q, kp, vp, bt, c, cu = _paged(rng, 1, 1, 1, d, [S], [k])
    out = oracle.spec_verify_attn(q, kp, vp, bt, c, cu, 0.5, draft_mask=np.array([1 << i for i in range(k)]))
    for i in range(k):
        keys = list(range(S)) + [S + i]
        sc = [0.5 * sum(q[i, 0, e] * kp[bt[0][p // PAGE], 0, p % PAGE, e] for e in range(d)) for p in keys]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        z = sum(w)
        for e in range(d):
            want = sum(w[j] * vp[bt[0][p // PAGE], 0, p % PAGE, e] for j, p in enumerate(keys)) / z
            assert abs(out[i, 0, e] - want) < 1e-12


def _tree_logits(rng, parents, V, p_match, distinct=False):
    """Random rows plus drafts that copy their parent row's argmax with prob p_match."""
    k = len(parents)
    logits = rng.standard_normal((k + 1, V)).astype(np.float32)
    t = np.argmax(logits, axis=1)
    drafts = []
    used = {}
    for i, p in enumerate(parents):
        want = int(t[p + 1])
        taken = used.setdefault(p, set())
        if rng.random() < p_match and not (distinct and want in taken):
            tok = want
        else:
            tok = int(rng.integers(0, V))
            while tok == want or (distinct and tok in taken):
                tok = int(rng.integers(0, V))
        taken.add(tok)
        drafts.append(tok)
    return logits, drafts


def test_chain_tree_equals_prefix_acceptance():
    rng = np.random.default_rng(5)
    for trial in range(40):
        ks = [int(rng.integers(0, 9)) for _ in range(3)]
        cu = np.concatenate([[0], np.cumsum(ks)])
        rows, drafts, parents = [], [], []
        for k in ks:
            par = [-1] + list(range(k - 1)) if k else []
            lg, dr = _tree_logits(rng, par, 50, 0.7)
            rows.append(lg)
            drafts += dr
            parents += par
        logits = np.concatenate(rows)
        t1, n1, x1 = oracle.accept_prefix(logits, np.array(drafts), cu)
        t2, n2, x2, path = oracle.accept_tree(logits, np.array(drafts), np.array(parents), cu)
        assert np.array_equal(t1, t2) and np.array_equal(n1, n2) and np.array_equal(x1, x2)
        for b in range(3):
            assert list(path[cu[b]:cu[b] + n1[b]]) == list(range(n1[b]))
            assert all(path[cu[b] + n1[b]:cu[b + 1]] == -1)


def test_tree_acceptance_matches_path_enumeration():
    """With distinct sibling tokens the accepted branch is the unique longest
    root-to-node path whose every draft equals the argmax of its parent's row."""
    rng = np.random.default_rng(8)
    for trial in range(200):
        k = int(rng.integers(1, 13))
        par = random_parents(rng, k, p_chain=0.4)
        logits, drafts = _tree_logits(rng, par, 7, 0.75, distinct=True)
        t = np.argmax(logits, axis=1)
        best = []
        for i in range(k):                       # path root -> i
            chain, j = [], i
            while j >= 0:
                chain.append(j)
                j = par[j]
            chain.reverse()
            ok = all(drafts[n] == t[par[n] + 1] for n in chain)
            if ok and len(chain) > len(best):
                best = chain
        _, n, nxt, path = oracle.accept_tree(logits, np.array(drafts), np.array(par), [0, k])
        assert n[0] == len(best) and list(path[:n[0]]) == best
        last = best[-1] if best else -1
        assert nxt[0] == t[last + 1]


def test_tree_acceptance_duplicate_siblings_take_lowest_index():
    V = 5
    logits = np.zeros((5, V), np.float32)
    logits[0, 2] = 1          # root row: token 2
    logits[2, 3] = 1          # after node 1: token 3
    logits[3, 4] = 1          # after node 2: token 4
    logits[4, 1] = 1          # after node 3: token 1
    parents = [-1, -1, 1, 0]  # nodes 0 and 1 both carry token 2; node 2 hangs off node 1
    drafts = [0, 2, 3, 2]     # node 0 does not match; node 1 matches, then node 2
    _, n, nxt, path = oracle.accept_tree(logits, np.array(drafts), np.array(parents), [0, 4])
    assert n[0] == 2 and list(path[:2]) == [1, 2] and nxt[0] == 4
    drafts = [2, 2, 3, 1]     # both roots carry 2: the lowest index (node 0) wins, node 3 (child
    _, n, nxt, path = oracle.accept_tree(logits, np.array(drafts), np.array(parents), [0, 4])
    assert n[0] == 1 and list(path[:1]) == [0]        # of node 0) carries 1, row 1 says 0
    assert nxt[0] == 0


def test_commit_identity_path_keeps_pool():
    rng = np.random.default_rng(4)
    q, kp, vp, bt, c, cu = _paged(rng, 2, 2, 2, 8, [7, 30], [4, 6])
    n = np.array([3, 6])
    path = np.array([0, 1, 2, -1, 0, 1, 2, 3, 4, 5])
    assert np.array_equal(oracle.commit_path(kp, bt, c, cu, n, path), kp)
    sc = rng.standard_normal(kp.shape[:3]).astype(np.float16)
    p2, s2 = oracle.commit_path(kp, bt, c, cu, n, path, scale=sc)
    assert np.array_equal(p2, kp) and np.array_equal(s2, sc)


def test_commit_turns_tree_attention_into_causal():
    """The deepest accepted node's tree-attention output equals causal
    attention after the branch is committed, for the same query."""
    rng = np.random.default_rng(12)
    for trial in range(10):
        S, k, d, H = int(rng.integers(0, 40)), int(rng.integers(2, 12)), 16, 2
        q, kp, vp, bt, c, cu = _paged(rng, 1, H, H, d, [S], [k])
        par = random_parents(rng, k)
        masks = oracle.ancestor_masks(np.array(par), cu)
        # accepted branch: root -> the last node
        chain, j = [], k - 1
        while j >= 0:
            chain.append(j)
            j = par[j]
        chain.reverse()
        n = len(chain)
        path = np.array(chain + [-1] * (k - n))
        tree = oracle.spec_verify_attn(q, kp, vp, bt, c, cu, 0.3, draft_mask=masks)
        kc = oracle.commit_path(kp, bt, c, cu, np.array([n]), path)
        vc = oracle.commit_path(vp, bt, c, cu, np.array([n]), path)
        q2 = np.zeros((n, H, d))
        q2[n - 1] = q[k - 1]
        causal = oracle.spec_verify_attn(q2, kc, vc, bt, c, np.array([0, n]), 0.3)
        np.testing.assert_allclose(causal[n - 1], tree[k - 1], rtol=1e-12, atol=1e-13)
        # rows outside the committed branch's span are untouched
        for p in range(S):
            pg, sl = bt[0][p // PAGE], p % PAGE
            assert np.array_equal(kc[pg, :, sl], kp[pg, :, sl])
