"""Oracle: the KV-cache management unit's pointer state machine.

Test infrastructure only (see the package docstring).

"HeteroReason", section on the KV Cache Management Unit (Fig. 7): three
pointer registers track the cache of each sequence -- Ptr_valid (the last
verified context boundary), Ptr_curr (the step under verification) and
Ptr_ahead (the step-ahead speculation frontier) -- and the controller runs in
four modes:

  Initialization  all three pointers are set to a given position (the prompt,
                  or the position a backtrack reverts to)
  Speculation     Ptr_valid and Ptr_curr stay; Ptr_ahead advances by the number
                  of speculative entries cached
  Accept          Ptr_valid <- Ptr_curr, Ptr_curr <- Ptr_ahead
  Rollback        Ptr_curr and Ptr_ahead <- Ptr_valid (the speculative history
                  is discarded by the pointer move alone)

Token-level verification (the blog's acceptance, and this library's accept
calls) accepts a prefix of n_b drafts rather than a whole step.  Reading used
here: a fifth mode, Prefix commit, accepts the first n_b entries after
Ptr_valid and rolls back the rest -- Ptr_valid <- min(Ptr_valid + n_b,
Ptr_ahead), then Ptr_curr, Ptr_ahead <- Ptr_valid.

Modes are per sequence; ``arg`` is the position (Initialization), the count
(Speculation, Prefix commit) or unused.  Negative counts are read as 0.
"""
import numpy as np

INIT, SPECULATE, ACCEPT, ROLLBACK, PREFIX = 0, 1, 2, 3, 4


def kvmu_apply(state, mode, arg):
    """state [B, 3] (valid, curr, ahead), mode [B], arg [B] -> new state [B, 3]."""
    out = np.array(state, dtype=np.int64).copy()
    for b in range(out.shape[0]):
        valid, curr, ahead = (int(x) for x in out[b])
        m, a = int(mode[b]), int(arg[b])
        if m == INIT:
            valid = curr = ahead = a
        elif m == SPECULATE:
            ahead = ahead + max(a, 0)
        elif m == ACCEPT:
            valid, curr = curr, ahead
        elif m == ROLLBACK:
            curr = ahead = valid
        elif m == PREFIX:
            valid = min(valid + max(a, 0), ahead)
            curr = ahead = valid
        out[b] = (valid, curr, ahead)
    return out


# ---------------------------------------------------------------------------
# Pages of the speculative history
# ---------------------------------------------------------------------------
#
# The same section: rejected speculative history is discarded by moving the
# pointers alone.  Reading used here for the pages that history occupied: once
# a sequence's valid pointer is final for the step, every page of its block
# table that lies wholly at or past it (logical page j with 16 j >= valid)
# holds nothing valid, so it goes back to the caller's free list and its entry
# becomes -1.  Before the next step writes rows at positions S_b .. S_b+k_b-1,
# each unassigned logical page those positions (or any earlier one) fall in
# takes a page from the top of the free list.  Orders are fixed so that the
# result is one definite array: pages are returned sequence by sequence,
# logical page by logical page, appended after the list's current entries;
# they are taken in the same order, each from the current top of the list.
# A list with too few pages leaves the remaining entries -1; a full list keeps
# counting (entries past its capacity are not stored).

def reclaim_pages(block_table, valid_lens, free_list, free_count, page=16):
    """Returns (block_table, free_list, free_count) after returning every page
    wholly at or past valid_lens[b] of every sequence b.  Entries < 0 are
    unassigned and stay so.  free_list is a 1-D array (its length is the
    capacity); free_count the number of entries in use."""
    bt = np.array(block_table, dtype=np.int64).copy()
    fl = np.array(free_list, dtype=np.int64).copy()
    count = int(free_count)
    B, max_pages = bt.shape
    for b in range(B):
        valid = max(int(valid_lens[b]), 0)
        for j in range(max_pages):
            if page * j >= valid and bt[b, j] >= 0:
                if count < len(fl):
                    fl[count] = bt[b, j]
                count += 1
                bt[b, j] = -1
    return bt, fl, count


def alloc_pages(block_table, ctx_lens, cu_q, free_list, free_count, page=16):
    """Returns (block_table, free_count) after giving every unassigned logical
    page j with 16 j < S_b + k_b (k_b = cu_q[b+1] - cu_q[b]) a page taken
    from the top of the free list (free_list[free_count - 1] first)."""
    bt = np.array(block_table, dtype=np.int64).copy()
    count = int(free_count)
    B, max_pages = bt.shape
    for b in range(B):
        end = max(int(ctx_lens[b]), 0) + max(int(cu_q[b + 1]) - int(cu_q[b]), 0)
        for j in range(max_pages):
            if page * j < end and bt[b, j] < 0 and count > 0:
                count -= 1
                bt[b, j] = int(free_list[count])
    return bt, count
