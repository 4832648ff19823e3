"""GPU parity of sva_accept_stochastic against the fp64 oracle (through the C ABI).

The GPU takes its decisions in fp32, the oracle in fp64; where a uniform lies
within rounding of p(x)/q(x), or u_sample * total within rounding of a
running-sum boundary, either neighbouring outcome is correct.  The parity
cases therefore move every uniform that the oracle finds closer than 1e-4
(relative) to a boundary out of that band first, then require bit-exact
accept lengths and tokens.  One large case keeps its raw uniforms and checks
validity instead: every GPU decision either matches the oracle or sits in the
ambiguous band, and the emitted token lies in the support with its running-sum
interval containing u * total up to rounding.  Also: the page's worked example
and the greedy limit (near-zero temperature equals greedy acceptance).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import token_verify_attention_amd as tva
from oracle.stochastic import softmax_t
from token_verify_attention_amd import workloads as wl
from gpu_helpers import np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BAND = 1e-4


def _case(ks, V, match, ident, noise=0.5, temperature=1.0, seed=0):
    w = wl.Workload("s", 1, 4, 4, 64, 0, 1, "f32", "f32", 1.0, V, match, False, ident)
    case = wl.make_case(w, device=DEV, ctx=[3] * len(ks), k=ks)
    case["draft_logits"] = wl.make_draft_logits(case["logits"], ks, device=DEV, seed=seed,
                                                noise=noise)
    ua, us = wl.make_uniforms(case["T"], case["B"], device=DEV, seed=seed)
    case["u_accept"], case["u_sample"] = ua, us
    return case


def _batch(case):
    return tva.Batch(case["ctx_lens"], case["cu_q"], total_q=case["T"], max_q=case["max_q"],
                     max_len=case["max_len"])


def _oracle(case, temperature, ua=None, us=None):
    return oracle.accept_stochastic(np_(case["logits"]), np_(case["draft_logits"]),
                                    np_(case["draft_ids"]), np_(case["cu_q"]), temperature,
                                    np_(case["u_accept"]) if ua is None else ua,
                                    np_(case["u_sample"]) if us is None else us,
                                    return_details=True)


def _unambiguous(case, temperature):
    """Move uniforms out of the rounding band around the oracle's boundaries."""
    ua, us = np_(case["u_accept"]).astype(np.float64), np_(case["u_sample"]).astype(np.float64)
    _, _, det = _oracle(case, temperature, ua, us)
    r = det["ratio"]
    for j in range(len(ua)):
        if np.isfinite(r[j]) and abs(ua[j] - r[j]) <= BAND * max(1.0, r[j]):
            ua[j] = (r[j] + 0.01) % 1.0
    n, _, det = _oracle(case, temperature, ua, us)
    for b, w in det["sample_weights"].items():
        cdf = np.cumsum(w) / w.sum()
        while np.abs(cdf - us[b]).min() <= BAND:
            us[b] = (us[b] + 0.0137) % 1.0
    ua32, us32 = ua.astype(np.float32), us.astype(np.float32)
    case["u_accept"] = torch.tensor(ua32, device=DEV)
    case["u_sample"] = torch.tensor(us32, device=DEV)
    return ua32.astype(np.float64), us32.astype(np.float64)


@pytest.mark.parametrize("V,match,temp", [(1000, 0.8, 1.0), (128256, 0.8, 1.0), (37, 0.5, 0.7),
                                          (4096, 0.9, 2.0), (50000, 0.3, 0.5)])
def test_parity_bit_exact(V, match, temp):
    ks = [4, 8, 1, 0, 16, 3, 7, 2]
    case = _case(ks, V, match, ident=90 + V % 7, seed=V % 11)
    ua, us = _unambiguous(case, temp)
    say(f"stochastic parity V={V} T={temp}")
    n, tok = tva.accept_stochastic(_batch(case), case["logits"], case["draft_logits"],
                                   case["draft_ids"], case["u_accept"], case["u_sample"],
                                   temperature=temp)
    torch.cuda.synchronize()
    rn, rt, _ = _oracle(case, temp, ua, us)
    assert np.array_equal(np_(n), rn)
    assert np.array_equal(np_(tok), rt)


def test_worked_example_from_the_page():
    """p = [.5, .3, .2], q = [.2, .7, .1], "hello" drafted: accepted iff
    u < 3/7; a rejection emits "hi" for u_sample < .75, else "hey"."""
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.2, 0.7, 0.1])
    case = _case([1], 3, 1.0, ident=95)
    case["logits"] = torch.tensor(np.log([p, p]), dtype=torch.float32, device=DEV)
    case["draft_logits"] = torch.tensor(np.log([q]), dtype=torch.float32, device=DEV)
    case["draft_ids"] = torch.tensor([1], dtype=torch.int32, device=DEV)
    b = _batch(case)
    out = []
    for ua, us in ((0.40, 0.5), (0.45, 0.5), (0.45, 0.74), (0.45, 0.76), (0.99, 0.9)):
        n, t = tva.accept_stochastic(b, case["logits"], case["draft_logits"], case["draft_ids"],
                                     torch.tensor([ua], device=DEV), torch.tensor([us], device=DEV))
        torch.cuda.synchronize()
        out.append((int(n[0]), int(t[0])))
    assert out[0][0] == 1                     # accepted: +1 token sampled from p
    assert out[1] == (0, 0) and out[2] == (0, 0) and out[3] == (0, 2) and out[4] == (0, 2)


def test_near_zero_temperature_equals_greedy():
    ks = [4, 8, 1, 16, 3]
    case = _case(ks, 2000, 0.6, ident=96)
    # a clear maximum in every target and drafter row
    lg = case["logits"]
    top = lg.argmax(dim=1)
    lg[torch.arange(lg.shape[0], device=DEV), top] += 1.0
    dl = case["draft_logits"]
    dl[torch.arange(dl.shape[0], device=DEV), case["draft_ids"].long()] = dl.max(dim=1).values + 1.0
    b = _batch(case)
    n, t = tva.accept_stochastic(b, lg, dl, case["draft_ids"], case["u_accept"], case["u_sample"],
                                 temperature=1e-4)
    _, gn, gt = tva.accept_prefix(b, lg, case["draft_ids"])
    torch.cuda.synchronize()
    assert torch.equal(n, gn) and torch.equal(t, gt)


def test_validity_with_raw_uniforms_full_size():
    """The ragged serving shape (vocabulary 128256) with unmodified uniforms."""
    w = wl.WORKLOADS["ragged_sampled"]
    case = wl.make_case(w, device=DEV)
    ks = case["k_host"]
    case["draft_logits"] = wl.make_draft_logits(case["logits"], ks, device=DEV, seed=w.ident)
    case["u_accept"], case["u_sample"] = wl.make_uniforms(case["T"], case["B"], device=DEV,
                                                          seed=w.ident)
    say("stochastic full size")
    n, tok = tva.accept_stochastic(_batch(case), case["logits"], case["draft_logits"],
                                   case["draft_ids"], case["u_accept"], case["u_sample"])
    torch.cuda.synchronize()
    n, tok = np_(n), np_(tok)
    ua, us = np_(case["u_accept"]).astype(np.float64), np_(case["u_sample"]).astype(np.float64)
    rn, rt, det = _oracle(case, 1.0, ua, us)
    r, cu = det["ratio"], np_(case["cu_q"])
    lg, dl = np_(case["logits"]), np_(case["draft_logits"])
    exact = 0
    for b in range(case["B"]):
        q0 = int(cu[b])
        # decisions up to the first disagreement must agree unless ambiguous
        for j in range(min(n[b], rn[b]) + (1 if n[b] != rn[b] else 0)):
            if j >= ks[b]:
                break
            gpu_acc = j < n[b]
            if gpu_acc != (ua[q0 + j] < r[q0 + j]):
                assert abs(ua[q0 + j] - r[q0 + j]) <= BAND * max(1.0, r[q0 + j])
        # the emitted token: support and running-sum interval of the row the GPU sampled
        row0 = q0 + b
        p = softmax_t(lg[row0 + n[b]], 1.0)
        wgt = np.maximum(p - softmax_t(dl[q0 + n[b]], 1.0), 0.0) if n[b] < ks[b] else p
        if not wgt.sum() > 0:
            wgt = p
        c = np.cumsum(wgt) / wgt.sum()
        v = int(tok[b])
        assert wgt[v] > 0
        lo, hi = (c[v - 1] if v else 0.0), c[v]
        assert lo - BAND <= us[b] <= hi + BAND
        exact += int(n[b] == rn[b] and tok[b] == rt[b])
    assert exact >= case["B"] - 2
