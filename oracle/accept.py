"""Oracle: greedy longest-prefix acceptance over the target's logits.

Test infrastructure only (see the package docstring).

"Decoding Speculative Decoding from First Principles", section "Speculating to
get sequence parallelism during decode": the target scores every draft in one
pass; at the first disagreement the draft is rejected and the target's own
token kept; the last row of the pass predicts the token after the last draft,
so one pass yields between 1 and n+1 tokens.

Greedy reading: the target's token at a row is the argmax of its logits.
Sequence b owns k_b + 1 logit rows starting at cu_q[b] + b; row j scores the
token after draft j-1 (row 0: after the committed context).  Ties go to the
lowest index; a NaN counts as the largest value and the first NaN wins (the
numpy convention; the page names no rule for ties or NaN).  -0.0 equals +0.0.
"""
import numpy as np


def argmax_rows(logits):
    """logits [R, V] float32 -> int64 [R]: first index of the row maximum."""
    logits = np.asarray(logits, dtype=np.float32)
    out = np.empty(logits.shape[0], dtype=np.int64)
    for r, row in enumerate(logits):
        nan_at = np.flatnonzero(np.isnan(row))
        if nan_at.size:
            out[r] = nan_at[0]
            continue
        out[r] = np.flatnonzero(row == row.max())[0]
    return out


def accept_prefix(logits, draft_ids, cu_q):
    """logits [T+B, V] float32, draft_ids [T] int, cu_q [B+1].

    Returns (argmax_ids [T+B], accept_len [B], next_token [B]) as int64.
    accept_len[b] = n, the number of leading drafts equal to the target's
    tokens; next_token[b] = the target's token at row n (the correction when a
    draft was rejected, the bonus token when all k_b were accepted).
    """
    cu_q = np.asarray(cu_q)
    B = len(cu_q) - 1
    t = argmax_rows(logits)
    accept_len = np.zeros(B, dtype=np.int64)
    next_token = np.zeros(B, dtype=np.int64)
    for b in range(B):
        q0 = int(cu_q[b])
        k = int(cu_q[b + 1]) - q0
        row0 = q0 + b
        n = 0
        while n < k and int(draft_ids[q0 + n]) == int(t[row0 + n]):
            n += 1
        accept_len[b] = n
        next_token[b] = t[row0 + n]
    return t, accept_len, next_token
