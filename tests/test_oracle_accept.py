"""Pins for the acceptance oracle (CPU only).

"Decoding Speculative Decoding from First Principles", section "Speculating to
get sequence parallelism during decode": reject at the first disagreement,
keep the target's token, the last row is the +1 bonus token, so each pass
yields 1 to n+1 tokens.  Pins: numpy.argmax as an independent library routine,
constructed tie / NaN / signed-zero / infinity rows, constructed acceptance
cases, and the generator's expected accept length sum_i p**i.
"""
import numpy as np
import pytest
import torch

import oracle
from token_verify_attention_amd import workloads


def test_argmax_matches_numpy_on_random_rows():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 777)).astype(np.float32)
    x[3, 100] = x[3, 50] = 9.0                       # duplicated maximum
    x[7, 5] = np.nan                                 # NaN wins
    x[7, 2] = np.nan
    assert np.array_equal(oracle.argmax_rows(x), np.argmax(x, axis=1))


def test_argmax_constructed_rows():
    neg = -np.ones(8, np.float32)
    r_tie = neg.copy(); r_tie[[2, 5, 6]] = 3.0
    r_zero = neg.copy(); r_zero[4] = -0.0; r_zero[1] = 0.0
    r_zero2 = neg.copy(); r_zero2[1] = -0.0; r_zero2[4] = 0.0
    r_inf = neg.copy(); r_inf[6] = np.inf; r_inf[3] = np.inf
    r_nan = neg.copy(); r_nan[6] = np.nan; r_nan[0] = np.inf
    r_neginf = np.full(8, -np.inf, np.float32)
    x = np.stack([r_tie, r_zero, r_zero2, r_inf, r_nan, r_neginf])
    assert list(oracle.argmax_rows(x)) == [2, 1, 1, 3, 6, 0]


def _logits_with_targets(targets, V=10):
    x = np.zeros((len(targets), V), np.float32)
    for r, t in enumerate(targets):
        x[r, t] = 1.0
    return x


def test_acceptance_constructed_cases():
    # b0: k=3 all drafts match -> n=3, next = bonus row's argmax
    # b1: k=2 first draft wrong -> n=0, next = row 0's argmax
    # b2: k=4 third draft wrong -> n=2, next = row 2's argmax
    # b3: k=0 -> n=0, next = its single row's argmax
    targets = [1, 2, 3, 9,   4, 5, 6,   7, 8, 0, 1, 2,   5]
    drafts = [1, 2, 3,   3, 5,   7, 8, 9, 1]
    cu = np.array([0, 3, 5, 9, 9])
    t, n, nxt = oracle.accept_prefix(_logits_with_targets(targets), np.array(drafts), cu)
    assert list(t) == targets
    assert list(n) == [3, 0, 2, 0]
    assert list(nxt) == [9, 4, 0, 5]
    emitted = n + 1
    assert ((emitted >= 1) & (emitted <= np.diff(cu) + 1)).all()


def test_generator_expected_accept_length():
    # E[n] = sum_{i=1..k} p**i for independent per-position agreement p.
    w = workloads.Workload("stat", 600, 1, 1, 8, 0, 4, "f32", "f32", 1.0, 64, 0.7, False, 99)
    lg = workloads.make_logits(w, [4] * w.B, device="cpu")
    cu = np.arange(0, 4 * w.B + 1, 4)
    t, n, _ = oracle.accept_prefix(lg["logits"].numpy(), lg["draft_ids"].numpy(), cu)
    assert np.array_equal(t, lg["planted"].numpy())
    expect = sum(0.7 ** i for i in range(1, 5))                 # 1.7731
    var = np.var(n)
    assert abs(n.mean() - expect) < 4 * np.sqrt(var / w.B)


def test_planted_rows_put_the_maximum_where_planted():
    g = torch.Generator().manual_seed(0)
    planted = torch.randint(0, 5000, (16,), generator=g)
    rows = workloads.planted_rows(16, 5000, planted, g, "cpu")
    assert torch.equal(rows.argmax(dim=1), planted)
    # the marginal law is N(0,1): mean ~ 0, var ~ 1 over 80k draws
    assert abs(rows.mean().item()) < 0.02 and abs(rows.var().item() - 1) < 0.03
