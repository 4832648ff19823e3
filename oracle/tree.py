"""Oracle: tree-structured verification (token trees).

Test infrastructure only (see the package docstring).

"Decoding Speculative Decoding from First Principles", section "Tree based
verification" (SpecInfer, EAGLE-2, DDTree): instead of one draft sequence the
drafter proposes a tree of continuations; the target checks every branch in
the same pass with "tree attention", in which a draft relates only to its own
lineage back to the committed context; the accepted continuation is the
longest branch the target agrees with.

The page gives no formulas.  Readings used here (and by the library):

* A tree of k_b nodes is a parent array in topological order:
  parent[i] = -1 (a child of the last committed token) or 0 <= parent[i] < i.
* Node i's K/V row sits at logical position S_b + i.  Node i attends to the
  committed context (positions 0 .. S_b-1) and to the nodes of its lineage:
  itself and its ancestors.  As a bitmask over the sequence's nodes that is
  ancestor_masks()[i]; the attention oracle takes such masks (bit j: node j is
  visible), so a chain (parent[i] = i-1) gives the causal draft mask.
* Greedy acceptance: logit row 0 of the sequence scores the token after the
  committed context, row 1 + i the token after node i (the chain layout).
  Starting at the root, the target's token t is the argmax of the current
  row; the walk moves to the child whose draft token equals t (the lowest
  index when several children carry t) and stops when no child does.  The
  step emits the path's draft tokens and then t: n_b + 1 tokens.
* Commit: the accepted path's K/V rows move to positions S_b .. S_b+n_b-1, so
  the cache holds one linear sequence again ("HeteroReason", KVMU: rejected
  speculative history is discarded by a pointer rollback; here the surviving
  branch is first made contiguous).
"""
import numpy as np

from .accept import argmax_rows


def ancestor_masks(parents, cu_q):
    """parents [T] int (per sequence, -1 or an earlier node index), cu_q [B+1].

    Returns int64 [T]: bit j of entry cu_q[b] + i is set when node j of
    sequence b is node i or one of its ancestors.  Out-of-range parents
    (>= i or < -1) are read as -1.
    """
    parents = np.asarray(parents)
    cu_q = np.asarray(cu_q)
    out = np.zeros(len(parents), dtype=np.int64)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        for i in range(q1 - q0):
            m, j = 0, i
            while j >= 0:
                m |= 1 << j
                pj = int(parents[q0 + j])
                j = pj if 0 <= pj < j else -1
            out[q0 + i] = m
    return out


def accept_tree(logits, draft_ids, parents, cu_q):
    """Greedy tree acceptance.

    logits [T+B, V] float32, draft_ids [T], parents [T], cu_q [B+1].
    Returns (argmax_ids [T+B], accept_len [B], next_token [B], accept_path [T])
    as int64; accept_path holds, per sequence, the accepted nodes in path
    order followed by -1.
    """
    cu_q = np.asarray(cu_q)
    parents = np.asarray(parents)
    B = len(cu_q) - 1
    t = argmax_rows(logits)
    accept_len = np.zeros(B, dtype=np.int64)
    next_token = np.zeros(B, dtype=np.int64)
    path = -np.ones(len(draft_ids), dtype=np.int64)
    for b in range(B):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k = q1 - q0
        row0 = q0 + b
        cur, n = -1, 0
        while True:
            want = int(t[row0 + 1 + cur])          # row of the current node (root: row0)
            nxt = -1
            for c in range(k):
                pc = int(parents[q0 + c])
                pc = pc if 0 <= pc < c else -1
                if pc == cur and int(draft_ids[q0 + c]) == want:
                    nxt = c
                    break
            if nxt < 0:
                break
            path[q0 + n] = nxt
            n += 1
            cur = nxt
        accept_len[b] = n
        next_token[b] = t[row0 + 1 + cur]
    return t, accept_len, next_token, path


def commit_path(pool, block_table, ctx_lens, cu_q, accept_len, accept_path, scale=None):
    """Move the accepted path's rows to S_b .. S_b+n_b-1, every kv head.

    pool [P, Hkv, page, d] (values or INT8 codes), scale [P, Hkv, page] or None.
    Rows are read from the pool as it was before the call.  Returns the new
    pool (and the new scale array when one is given).
    """
    page = pool.shape[2]
    src_pool = pool
    new_pool = pool.copy()
    new_scale = None if scale is None else scale.copy()
    cu_q = np.asarray(cu_q)
    for b in range(len(cu_q) - 1):
        S, q0 = int(ctx_lens[b]), int(cu_q[b])
        for j in range(int(accept_len[b])):
            src = S + int(accept_path[q0 + j])
            dst = S + j
            ps, ss = int(block_table[b][src // page]), src % page
            pd, sd = int(block_table[b][dst // page]), dst % page
            new_pool[pd, :, sd, :] = src_pool[ps, :, ss, :]
            if scale is not None:
                new_scale[pd, :, sd] = scale[ps, :, ss]
    if scale is None:
        return new_pool
    return new_pool, new_scale
