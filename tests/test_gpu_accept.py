"""GPU parity of sva_accept_prefix against the oracle: argmax ids, accept
lengths and next tokens are bit-exact (lowest index on ties, first NaN wins,
-0.0 == +0.0)."""
import numpy as np
import pytest
import torch

import oracle
import token_verify_attention_amd as tva
from token_verify_attention_amd import workloads as wl
from gpu_helpers import batch_of, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run_and_compare(batch, logits, drafts, cu):
    ids, n, nxt = tva.accept_prefix(batch, logits, drafts)
    torch.cuda.synchronize()
    rt, rn, rx = oracle.accept_prefix(np_(logits), np_(drafts), cu)
    assert np.array_equal(np_(ids), rt)
    assert np.array_equal(np_(n), rn)
    assert np.array_equal(np_(nxt), rx)
    return rn


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_workload_acceptance(name):
    w = wl.WORKLOADS[name]
    say(f"accept {name}")
    case = wl.make_case(w, device=DEV)
    n = _run_and_compare(batch_of(case), case["logits"], case["draft_ids"], np_(case["cu_q"]))
    k = np.array(case["k_host"])
    assert ((n >= 0) & (n <= k)).all()


def _batch(ks, max_len=10):
    cu = torch.zeros(len(ks) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(ks), 0)
    ctx = torch.full((len(ks),), 5, dtype=torch.int32)
    return tva.Batch(ctx.to(DEV), cu.to(DEV), total_q=int(cu[-1]), max_q=max(max(ks), 1),
                     max_len=max_len + max(ks)), cu.numpy()


@pytest.mark.parametrize("V", [1000, 4099, 70001, 128256])
def test_constructed_rows(V):
    say(f"accept constructed V={V}")
    ks = [3, 2, 4, 0, 1, 16]
    batch, cu = _batch(ks)
    rows = sum(ks) + len(ks)
    g = torch.Generator(device=DEV).manual_seed(V)
    x = torch.randn((rows, V), generator=g, device=DEV)
    x[0, [7, V - 1, 5]] = 50.0                          # tie: lowest index wins
    x[1, :] = -1.0
    x[1, V // 2] = -0.0                                  # -0.0 == +0.0
    x[1, V // 3] = 0.0
    x[2, 11] = float("nan")                              # NaN wins, first NaN
    x[2, 3] = float("nan")
    x[2, 0] = float("inf")
    x[3, :] = float("-inf")                             # all -inf -> index 0
    x[4, [100 % V, V - 2]] = float("inf")
    # drafts: sequence 0 all match, 1 first wrong, 2 third wrong, 4 matches, 5 random
    t = oracle.argmax_rows(np_(x))
    d = []
    for b, k in enumerate(ks):
        row0 = cu[b] + b
        for j in range(k):
            tj = int(t[row0 + j])
            wrong = (b == 1 and j == 0) or (b == 2 and j == 2) or (b == 5 and j == 9)
            d.append((tj + 1) % V if wrong else tj)
    drafts = torch.tensor(d, dtype=torch.int32, device=DEV)
    n = _run_and_compare(batch, x, drafts, cu)
    assert list(n) == [3, 0, 2, 0, 1, 9]


def test_unaligned_vocab_scalar_path():
    ks = [2, 3]
    batch, cu = _batch(ks)
    V = 1001
    g = torch.Generator(device=DEV).manual_seed(5)
    big = torch.randn((sum(ks) + 2) * V + 1, generator=g, device=DEV)
    x = big[1:].view(sum(ks) + 2, V)                     # rows not 16-byte aligned
    drafts = torch.zeros(sum(ks), dtype=torch.int32, device=DEV)
    _run_and_compare(batch, x, drafts, cu)


def test_one_workspace_serves_calls_of_any_shape():
    """One workspace reused across batches, vocabularies and chunkings (the
    chunk keys of one call never leak into the next)."""
    shapes = [([3, 2, 4, 0, 1, 16], 128256), ([1], 1000), ([8] * 40, 4099),
              ([2, 5], 70001), ([16] * 3, 128256)]
    nmax = 0
    for ks, V in shapes:
        batch, _ = _batch(ks)
        nmax = max(nmax, tva.accept_workspace_bytes(batch, V))
    ws = torch.zeros(nmax, dtype=torch.uint8, device=DEV)
    for i, (ks, V) in enumerate(shapes * 2):
        say(f"accept workspace reuse {i}: B={len(ks)} V={V}")
        batch, cu = _batch(ks)
        g = torch.Generator(device=DEV).manual_seed(100 + i)
        x = torch.randn((sum(ks) + len(ks), V), generator=g, device=DEV)
        t = oracle.argmax_rows(np_(x))
        d = [int(t[cu[b] + b + j]) if (j + b) % 3 else (int(t[cu[b] + b + j]) + 1) % V
             for b, k in enumerate(ks) for j in range(k)]
        drafts = torch.tensor(d, dtype=torch.int32, device=DEV)
        ids, n, nxt = tva.accept_prefix(batch, x, drafts, workspace=ws)
        torch.cuda.synchronize()
        rt, rn, rx = oracle.accept_prefix(np_(x), np_(drafts), cu)
        assert np.array_equal(np_(ids), rt) and np.array_equal(np_(n), rn)
        assert np.array_equal(np_(nxt), rx)
