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


# ---- pages of the speculative history ---------------------------------------

from oracle.kvmu import alloc_pages, reclaim_pages   # noqa: E402


def test_reclaim_hand_worked():
    """Two sequences of four logical pages.  Sequence 0 keeps 20 rows: pages
    0 (rows 0-15) and 1 (rows 16-19, partly valid) stay, pages 2 and 3 go.
    Sequence 1 keeps 32 rows (exactly two pages): pages 2 (id 9) and 3
    (unassigned) -- only id 9 goes.  Appended after the list's 2 entries,
    sequence 0's pages first, in logical order."""
    bt = [[4, 7, 2, 5], [8, 1, 9, -1]]
    fl = np.full(8, -7)
    fl[:2] = [30, 31]
    nbt, nfl, n = reclaim_pages(bt, [20, 32], fl, 2)
    assert nbt.tolist() == [[4, 7, -1, -1], [8, 1, -1, -1]]
    assert nfl.tolist()[:5] == [30, 31, 2, 5, 9] and n == 5
    # a valid length of 0 frees everything; a length past the table frees nothing
    nbt, _, n = reclaim_pages(bt, [0, 1000], np.zeros(8), 0)
    assert nbt.tolist() == [[-1, -1, -1, -1], [8, 1, 9, -1]] and n == 4


def test_alloc_hand_worked():
    """Sequence 0: S=20, k=5 -> rows up to 24 -> pages 0 and 1 needed, page 1
    unassigned takes the list's top (id 12).  Sequence 1: S=31, k=3 -> rows up
    to 33 -> pages 0..2; pages 1 and 2 unassigned take 11 then 10."""
    bt = [[3, -1, -1, -1], [6, -1, -1, -1]]
    fl = [10, 11, 12]
    nbt, n = alloc_pages(bt, [20, 31], [0, 5, 8], fl, 3)
    assert nbt.tolist() == [[3, 12, -1, -1], [6, 11, 10, -1]] and n == 0
    # too few pages: the rest stay unassigned, the count stops at zero
    nbt, n = alloc_pages(bt, [20, 31], [0, 5, 8], [10], 1)
    assert nbt.tolist() == [[3, 10, -1, -1], [6, -1, -1, -1]] and n == 0


def test_pages_are_conserved_and_unique_over_a_random_loop():
    """Over many steps of alloc -> (random acceptance) -> reclaim, every page
    is either in exactly one block-table entry or on the free list, never
    both; rows below each valid length keep their pages; and after a reclaim
    no assigned page lies wholly past its sequence's valid length."""
    rng = np.random.default_rng(3)
    B, max_pages, P = 6, 40, 200
    lens = rng.integers(0, 300, B)
    bt = np.full((B, max_pages), -1)
    free = list(range(P))
    rng.shuffle(free)
    fl = np.array(free + [-1] * 50)
    count = P
    # initial contexts take their pages
    bt, count = alloc_pages(bt, lens, np.zeros(B + 1, int), fl, count)
    for _ in range(300):
        ks = rng.integers(0, 9, B)
        cu = np.concatenate([[0], np.cumsum(ks)])
        before = bt.copy()
        bt, count = alloc_pages(bt, lens, cu, fl, count)
        for b in range(B):
            for j in range(max_pages):
                if 16 * j < lens[b]:
                    assert bt[b, j] == before[b, j]      # valid rows never move
        n = np.array([rng.integers(0, k + 1) for k in ks])
        lens = lens + n
        if rng.random() < 0.1:
            lens = np.maximum(lens - rng.integers(0, 40, B), 0)   # a deeper rollback
        bt, fl, count = reclaim_pages(bt, lens, fl, count)
        assigned = bt[bt >= 0].tolist()
        listed = fl[:count].tolist()
        assert sorted(assigned + listed) == list(range(P))
        for b in range(B):
            for j in range(max_pages):
                if bt[b, j] >= 0:
                    assert 16 * j < lens[b]
