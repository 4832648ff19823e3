"""Oracle: lossless stochastic acceptance (speculative rejection sampling).

Test infrastructure only (see the package docstring).

"Decoding Speculative Decoding from First Principles", section "How does this
drafter maintain the same distribution of the target?": with p the target's
and q the drafter's distribution at a draft position and x the drafted token,
the draft is accepted with probability min(1, p(x)/q(x)) (always when
p(x) >= q(x), p/q of the time otherwise); on a rejection the token is sampled
from the residual max(p - q, 0), renormalised, and the pass stops.  The page's
proof shows the emitted token then has distribution p exactly.  When every
draft is accepted the pass still yields the target's next token, sampled from
p at the row after the last draft (the "+1" of the section on sequence
parallelism).

Readings (the page gives the rule, not an interface):
* Distributions are softmax(logits / temperature) of the target's and the
  drafter's logits, one temperature for both.
* Random numbers are inputs: u_accept[j] in [0, 1) decides draft j (accept
  iff u < p(x)/q(x)); u_sample[b] in [0, 1) samples sequence b's emitted
  token by inverse CDF: the first index whose running sum of the (unnormalised)
  weights exceeds u * their total.
* A residual that is zero everywhere (p = q, where a rejection has probability
  zero) samples from p instead.
"""
import numpy as np


def softmax_t(row, temperature):
    """softmax(row / temperature) in float64."""
    x = np.asarray(row, dtype=np.float64) / float(temperature)
    e = np.exp(x - x.max())
    return e / e.sum()


def sample_inverse_cdf(weights, u):
    """First index whose running sum of weights exceeds u * total."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    return int(np.searchsorted(c, u * c[-1], side="right"))


def accept_stochastic(target_logits, draft_logits, draft_ids, cu_q, temperature, u_accept,
                      u_sample, return_details=False):
    """target_logits [T+B, V] (rows as for greedy acceptance), draft_logits
    [T, V] (the drafter's logits at each draft position), draft_ids [T],
    cu_q [B+1], u_accept [T], u_sample [B].

    Returns (accept_len [B], next_token [B]) as int64, and with
    ``return_details`` a dict: ratio [T] (p(x)/q(x)), sample_weights {b: the
    unnormalised weights the emitted token was drawn from}.
    """
    cu_q = np.asarray(cu_q)
    B = len(cu_q) - 1
    accept_len = np.zeros(B, dtype=np.int64)
    next_token = np.zeros(B, dtype=np.int64)
    ratio = np.full(len(draft_ids), np.nan)
    weights = {}
    for b in range(B):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        row0 = q0 + b
        n = q1 - q0
        w = None
        for j in range(q1 - q0):
            p = softmax_t(target_logits[row0 + j], temperature)
            q = softmax_t(draft_logits[q0 + j], temperature)
            x = int(draft_ids[q0 + j])
            r = np.inf if q[x] == 0 else p[x] / q[x]
            ratio[q0 + j] = r
            if not float(u_accept[q0 + j]) < r:
                n = j
                w = np.maximum(p - q, 0.0)
                if not w.sum() > 0:
                    w = p
                break
        if w is None:                                  # every draft accepted: the +1 token
            w = softmax_t(target_logits[row0 + n], temperature)
        accept_len[b] = n
        next_token[b] = sample_inverse_cdf(w, float(u_sample[b]))
        weights[b] = w
    if return_details:
        return accept_len, next_token, dict(ratio=ratio, sample_weights=weights)
    return accept_len, next_token
