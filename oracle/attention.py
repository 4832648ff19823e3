"""Oracle: causal multi-query verification attention over a paged KV cache.

Test infrastructure only (see the package docstring).

Definition followed ("Decoding Speculative Decoding from First Principles",
section "Speculating to get sequence parallelism during decode", and its
prerequisites on causal masked attention; "CXL-SpecKV", key observation (1)):
the target model scores the k_b draft tokens of sequence b in one pass.  Draft
query i (0-based) sits at logical position S_b + i, so it attends to every
committed context row and to drafts 0..i: keys p in [0, S_b + i].

For every sequence b, query i, head h (kv head g = h // G, G = Hq / Hkv):

    K_p = deq(K_pool[block_table[b][p // page], g, p % page, :])
    s_p = scale * <q_{i,h}, K_p>          p = 0 .. S_b + i
    w_p = exp(s_p - max s) / sum exp(s - max s)
    out_{i,h} = sum_p w_p V_p

Tree-structured verification ("Decoding Speculative Decoding from First
Principles", section "Tree based verification": tree attention relates a draft
only to its own lineage) replaces the causal draft mask by a per-draft bitmask:
with ``draft_mask`` given, draft i sees the committed rows 0 .. S_b-1 and the
draft rows S_b + j (j < k_b) whose bit j is set in draft_mask[cu_q[b] + i].

All arithmetic is float64.  float32 / bf16 inputs and int8 codes times fp16
scales convert to float64 exactly, so the only rounding is the fp64 arithmetic
itself.
"""
import numpy as np


def _dequant(pool, scale, pages, g, slots):
    rows = pool[pages, g, slots, :].astype(np.float64)
    if scale is not None:
        rows = rows * scale[pages, g, slots].astype(np.float64)[:, None]
    return rows


def spec_verify_attn(q, k_pool, v_pool, block_table, ctx_lens, cu_q, softmax_scale,
                     k_scale=None, v_scale=None, select=None, return_weights=False,
                     draft_mask=None):
    """Plain-definition verification attention.

    q            [T, Hq, d] float (float32 values, or bf16 values held in float32)
    k_pool/v_pool [P, Hkv, page, d] float values, or int8 codes when the
                 matching ``*_scale`` [P, Hkv, page] float16 array is given
    block_table  [B, max_pages] int, physical page of each logical page
    ctx_lens     [B] committed rows S_b (the k_b draft rows come after them)
    cu_q         [B+1] prefix sums of k_b
    select       optional iterable of (b, g) pairs; other rows stay NaN
    draft_mask   optional [T] int bitmasks (tree attention; see module doc)
    Returns out [T, Hq, d] float64 (and, if asked, a dict mapping
    (b, i, h) -> the weight vector over the visible keys in position order).
    """
    q = np.asarray(q)
    T, Hq, d = q.shape
    _, Hkv, page, d2 = k_pool.shape
    assert d2 == d and Hq % Hkv == 0
    G = Hq // Hkv
    B = len(ctx_lens)
    out = np.full((T, Hq, d), np.nan, dtype=np.float64)
    weights = {} if return_weights else None
    pairs = [(b, g) for b in range(B) for g in range(Hkv)] if select is None else list(select)
    for b, g in pairs:
        S = int(ctx_lens[b])
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k = q1 - q0
        if k == 0:
            continue
        pos = np.arange(S + k)
        pages = np.asarray(block_table[b])[pos // page].astype(np.int64)
        slots = pos % page
        K = _dequant(k_pool, k_scale, pages, g, slots)   # [S+k, d]
        V = _dequant(v_pool, v_scale, pages, g, slots)
        for i in range(k):
            if draft_mask is None:
                Ki, Vi = K[:S + i + 1], V[:S + i + 1]      # keys 0 .. S+i
            else:
                m = int(draft_mask[q0 + i])
                keys = np.concatenate([np.arange(S),
                                       [S + j for j in range(k) if (m >> j) & 1]]).astype(np.int64)
                Ki, Vi = K[keys], V[keys]
            for j in range(G):
                h = g * G + j
                qv = q[q0 + i, h].astype(np.float64)
                s = float(softmax_scale) * (Ki @ qv)
                e = np.exp(s - s.max())
                w = e / e.sum()
                out[q0 + i, h] = w @ Vi
                if weights is not None:
                    weights[(b, i, h)] = w
    if return_weights:
        return out, weights
    return out
