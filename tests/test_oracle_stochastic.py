"""Pins for the stochastic-acceptance oracle (CPU only).

"Decoding Speculative Decoding from First Principles", section "How does this
drafter maintain the same distribution of the target?": accept the drafted
token with probability min(1, p/q), else sample the residual max(p - q, 0);
the emitted token is then distributed exactly as p.  Pins: the page's worked
example (tests/golden/rejection_example.txt), the distribution identity
checked exactly by locating the oracle's decision boundaries, the greedy
limit (near-zero temperature reproduces greedy prefix acceptance), and the
special cases p = q, q(x) = 0 and p(x) = 0.
"""
import os

import numpy as np
import pytest

import oracle
from oracle.stochastic import accept_stochastic, sample_inverse_cdf, softmax_t

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rejection_example.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        vals[k.strip()] = [float(x) for x in v.split()]
    return vals


def _one(p, q, x, u_a, u_s):
    """One sequence, one draft, logits log p / log q at temperature 1."""
    tl = np.log(np.array([p, p], dtype=np.float64)).astype(np.float64)   # row 0 and bonus row
    dl = np.log(np.array([q], dtype=np.float64))
    n, t = accept_stochastic(tl, dl, np.array([x]), np.array([0, 1]), 1.0, np.array([u_a]),
                             np.array([u_s]))
    return int(n[0]), int(t[0])


def _accept_boundary(p, q, x, iters=60):
    """Largest u_accept the oracle still accepts (bisection)."""
    lo, hi = 0.0, 1.0
    if _one(p, q, x, 0.0, 0.5)[0] == 0:
        return 0.0
    if _one(p, q, x, np.nextafter(1.0, 0.0), 0.5)[0] == 1:
        return 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if _one(p, q, x, mid, 0.5)[0] == 1:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _residual_cdf(p, q, x, iters=60):
    """The emitted-token CDF after a rejection, located by bisection on u_sample."""
    V = len(p)
    bounds = []
    for v in range(V - 1):                    # first u_s at which the token exceeds v
        lo, hi = 0.0, 1.0
        if _one(p, q, x, 0.999999999, 0.0)[1] > v:
            bounds.append(0.0)
            continue
        for _ in range(iters):
            mid = 0.5 * (lo + hi)
            if _one(p, q, x, 0.999999999, mid)[1] > v:
                hi = mid
            else:
                lo = mid
        bounds.append(0.5 * (lo + hi))
    cdf = np.array(bounds + [1.0])
    return np.diff(np.concatenate([[0.0], cdf]))


def test_worked_example_from_the_page():
    g = _golden()
    p, q, x = np.array(g["p"]), np.array(g["q"]), int(g["draft"][0])
    a = g["accept_probability"][0]
    assert abs(_accept_boundary(p, q, x) - a) < 1e-12
    assert abs(a - 3.0 / 7.0) < 1e-15
    res = _residual_cdf(p, q, x)
    np.testing.assert_allclose(res, g["residual"], atol=1e-12)
    # "likely hi": a rejection with u_sample below .75 emits "hi" (index 0)
    assert _one(p, q, x, 0.9, 0.5) == (0, 0)
    assert _one(p, q, x, 0.9, 0.8) == (0, 2)
    assert _one(p, q, x, 0.2, 0.8)[0] == 1


@pytest.mark.parametrize("seed", range(8))
def test_output_distribution_equals_target_exactly(seed):
    """P(emit v) = q(v) a(v) + (sum_x q(x) (1 - a(x))) r(v) must equal p(v),
    with a(x) and r located from the oracle's own decisions."""
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 6))
    p = rng.dirichlet(np.ones(V) * 0.7)
    q = rng.dirichlet(np.ones(V) * 0.7)
    a = np.array([_accept_boundary(p, q, x) for x in range(V)])
    np.testing.assert_allclose(a, np.minimum(1.0, p / q), atol=1e-12)
    x_rej = int(np.argmax(q - p))              # a token that can be rejected
    r = _residual_cdf(p, q, x_rej)
    emit = q * a + (q * (1 - a)).sum() * r
    np.testing.assert_allclose(emit, p, atol=1e-11)


def test_near_zero_temperature_is_greedy_acceptance():
    rng = np.random.default_rng(3)
    for trial in range(30):
        ks = [int(rng.integers(0, 7)) for _ in range(4)]
        cu = np.concatenate([[0], np.cumsum(ks)])
        T, B, V = int(cu[-1]), len(ks), 40
        # rows with a clear maximum (gap >= 0.5): at temperature 1e-4 softmax is one-hot
        tl = rng.standard_normal((T + B, V))
        top = rng.integers(0, V, T + B)
        tl[np.arange(T + B), top] = tl.max(axis=1) + 0.5 + rng.random(T + B)
        drafts = np.empty(T, np.int64)
        dl = rng.standard_normal((T, V))
        for b in range(B):
            for j in range(ks[b]):
                t = top[cu[b] + b + j]
                drafts[cu[b] + j] = t if rng.random() < 0.6 else (t + 1 + rng.integers(0, V - 1)) % V
        dl[np.arange(T), drafts] = dl.max(axis=1) + 0.5 + rng.random(T)   # greedy drafter
        n, tok = accept_stochastic(tl, dl, drafts, cu, 1e-4, rng.random(T), rng.random(B))
        _, gn, gt = oracle.accept_prefix(tl.astype(np.float32), drafts, cu)
        assert np.array_equal(n, gn) and np.array_equal(tok, gt)


def test_special_cases():
    p = np.array([0.1, 0.6, 0.3])
    # p = q: always accepted, the +1 token comes from p
    assert _accept_boundary(p, p, 1) == 1.0
    # q(x) = 0 is accepted (ratio +inf); p(x) = 0 is always rejected
    with np.errstate(divide="ignore"):
        tl = np.log(np.array([[0.5, 0.5, 0.0], [0.2, 0.3, 0.5]]))
        dl = np.log(np.array([[0.0, 1.0, 0.0]]))
    with np.errstate(divide="ignore"):
        n, _ = accept_stochastic(tl, dl, np.array([0]), [0, 1], 1.0, np.array([0.999]), np.array([0.5]))
    assert n[0] == 1
    # p(2) = 0 < q(2) = .5: rejected even at u = 0; the residual
    # max(p - q, 0) = (.5, 0, 0) emits token 0
    with np.errstate(divide="ignore"):
        dl = np.log(np.array([[0.0, 0.5, 0.5]]))
        n, t = accept_stochastic(tl, dl, np.array([2]), [0, 1], 1.0, np.array([0.0]),
                                 np.array([0.99]))
    assert n[0] == 0 and t[0] == 0
    # inverse CDF skips zero-weight tokens
    assert sample_inverse_cdf(np.array([0.2, 0.0, 0.8]), 0.2) == 2
    assert sample_inverse_cdf(np.array([0.2, 0.0, 0.8]), 0.19) == 0
    # no drafts: the emitted token is sampled from row 0
    tl = np.log(np.array([[0.25, 0.75]]))
    n, t = accept_stochastic(tl, np.zeros((0, 2)), np.zeros(0, np.int64), [0, 0], 1.0,
                             np.zeros(0), np.array([0.3]))
    assert n[0] == 0 and t[0] == 1


def test_temperature_scales_logits():
    x = np.array([1.0, 2.0, 4.0])
    np.testing.assert_allclose(softmax_t(x, 2.0), softmax_t(x / 2.0, 1.0), rtol=1e-15)
    np.testing.assert_allclose(softmax_t(x, 1.0), np.exp(x) / np.exp(x).sum(), rtol=1e-14)
