"""Pins for the KVMU pointer state machine (CPU only).

"HeteroReason", KV Cache Management Unit (Fig. 7): the mode table is written
out below from the page's description (expected pointer triplets for each
mode), and invariants that follow from it are checked on random mode
sequences: valid <= curr <= ahead is preserved, Speculation never moves the
verified boundaries, Rollback returns curr and ahead to valid, and a step that
is speculated and then accepted twice in a row moves the verified boundary to
the old frontier.  The token-level Prefix commit is pinned against its
composition from the page's modes.
"""
import numpy as np

from oracle.kvmu import ACCEPT, INIT, PREFIX, ROLLBACK, SPECULATE, kvmu_apply

# (state before, mode, arg) -> state after, as the page describes each mode
TABLE = [
    ((5, 9, 14), INIT, 100, (100, 100, 100)),        # reset to a given position
    ((100, 120, 135), SPECULATE, 7, (100, 120, 142)),  # only the frontier moves
    ((100, 120, 135), ACCEPT, 0, (120, 135, 135)),   # valid <- curr, curr <- ahead
    ((100, 120, 135), ROLLBACK, 0, (100, 100, 100)),  # curr, ahead <- valid
    ((100, 100, 108), PREFIX, 3, (103, 103, 103)),   # keep 3 of 8, drop the rest
    ((100, 100, 108), PREFIX, 8, (108, 108, 108)),   # all accepted
    ((100, 100, 108), PREFIX, 20, (108, 108, 108)),  # never past the frontier
    ((100, 100, 108), PREFIX, -4, (100, 100, 100)),  # negative counts read as 0
    ((100, 100, 108), SPECULATE, -2, (100, 100, 108)),
]


def test_mode_table():
    for before, mode, arg, after in TABLE:
        got = kvmu_apply(np.array([before]), [mode], [arg])[0]
        assert tuple(got) == after, (before, mode, arg)


def test_modes_are_per_sequence():
    before = [(b, b, b) for b in (10, 20, 30, 40, 50)]
    mode = [INIT, SPECULATE, ACCEPT, ROLLBACK, PREFIX]
    got = kvmu_apply(np.array(before), mode, [7, 7, 7, 7, 7])
    assert [tuple(x) for x in got] == [(7, 7, 7), (20, 20, 27), (30, 30, 30), (40, 40, 40),
                                       (50, 50, 50)]


def test_invariants_on_random_sequences():
    rng = np.random.default_rng(1)
    B = 16
    st = kvmu_apply(np.zeros((B, 3)), [INIT] * B, rng.integers(0, 1000, B))
    for _ in range(500):
        mode = rng.integers(0, 5, B)
        arg = rng.integers(-3, 20, B)
        mode[mode == INIT] = SPECULATE if rng.random() < 0.9 else INIT
        new = kvmu_apply(st, mode, arg)
        assert (new[:, 0] <= new[:, 1]).all() and (new[:, 1] <= new[:, 2]).all()
        spec = mode == SPECULATE
        assert (new[spec, :2] == st[spec, :2]).all()
        rb = mode == ROLLBACK
        assert (new[rb, 1] == st[rb, 0]).all() and (new[rb, 2] == st[rb, 0]).all()
        acc = mode == ACCEPT
        assert (new[acc, 0] == st[acc, 1]).all() and (new[acc, 1] == st[acc, 2]).all()
        st = new


def test_step_ahead_accept_scenario():
    """Speculate a step, verify it while speculating the next one, accept
    twice: the verified boundary ends at the first step's frontier, then the
    second's."""
    s = kvmu_apply(np.array([(50, 50, 50)]), [SPECULATE], [12])     # step 1 drafted
    s = kvmu_apply(s, [ACCEPT], [0])                                 # curr <- 62 (verifying)
    assert tuple(s[0]) == (50, 62, 62)
    s = kvmu_apply(s, [SPECULATE], [9])                              # step-ahead drafting
    s = kvmu_apply(s, [ACCEPT], [0])                                 # step 1 verified
    assert tuple(s[0]) == (62, 71, 71)
    s = kvmu_apply(s, [ROLLBACK], [0])                               # step 2 rejected
    assert tuple(s[0]) == (62, 62, 62)


def test_prefix_commit_composes_page_modes():
    """Prefix commit of n = (curr - valid) entries from (v, v, a) equals
    Speculation up to curr, Accept, then Rollback of the step ahead."""
    rng = np.random.default_rng(2)
    for _ in range(200):
        v = int(rng.integers(0, 500))
        k = int(rng.integers(0, 17))
        n = int(rng.integers(0, k + 1))
        a = kvmu_apply(np.array([(v, v, v + k)]), [PREFIX], [n])[0]
        s = kvmu_apply(np.array([(v, v + n, v + k)]), [ACCEPT], [0])   # valid <- v + n
        s = kvmu_apply(s, [ROLLBACK], [0])
        assert tuple(a) == tuple(s[0])
