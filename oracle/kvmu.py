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
