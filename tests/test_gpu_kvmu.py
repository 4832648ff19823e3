"""GPU parity of sva_kvmu_apply against the KVMU oracle (through the C ABI):
random per-sequence mode sequences applied step by step (bit-exact pointer
triplets and ctx_lens), the uniform-mode form, and a three-step verification
loop whose committed lengths stay on the device: append -> attention ->
greedy acceptance -> Prefix commit, checked against the oracle's acceptance
and attention on the same inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import token_verify_attention_amd as tva
from oracle.kvmu import kvmu_apply as kvmu_ref
from token_verify_attention_amd import workloads as wl
from gpu_helpers import assert_close, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_random_mode_sequences_bit_exact():
    rng = np.random.default_rng(4)
    B = 300
    st_h = np.zeros((B, 3), np.int64)
    st = torch.zeros(B, 3, dtype=torch.int32, device=DEV)
    lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    say("kvmu random sequences")
    for step in range(60):
        mode = rng.integers(0, 6, B).astype(np.int32)          # 5 = unknown: no change
        arg = rng.integers(-3, 40, B).astype(np.int32)
        if step == 0:
            mode[:] = 0
            arg = rng.integers(0, 5000, B).astype(np.int32)
        tva.kvmu_apply(st, torch.tensor(mode, device=DEV), torch.tensor(arg, device=DEV), lens)
        known = mode < 5
        nxt = kvmu_ref(st_h, np.where(known, mode, 0), arg)
        st_h = np.where(known[:, None], nxt, st_h)
    torch.cuda.synchronize()
    assert np.array_equal(np_(st).astype(np.int64), st_h)
    assert np.array_equal(np_(lens).astype(np.int64), st_h[:, 0])


def test_uniform_modes():
    B = 5
    st = torch.tensor([[10, 12, 20]] * B, dtype=torch.int32, device=DEV)
    arg = torch.tensor([0, 1, 2, 3, 30], dtype=torch.int32, device=DEV)
    tva.kvmu_apply(st, tva.KVMU_PREFIX, arg)
    torch.cuda.synchronize()
    want = kvmu_ref(np.array([[10, 12, 20]] * B), [4] * B, np_(arg))
    assert np.array_equal(np_(st).astype(np.int64), want)
    tva.kvmu_apply(st, tva.KVMU_SPECULATE, arg)
    tva.kvmu_apply(st, tva.KVMU_ACCEPT)
    torch.cuda.synchronize()
    want = kvmu_ref(kvmu_ref(want, [1] * B, np_(arg)), [2] * B, [0] * B)
    assert np.array_equal(np_(st).astype(np.int64), want)


def test_verification_loop_commits_on_device():
    w = wl.Workload("loop", 1, 16, 4, 128, 0, 1, "bf16", "bf16", 1.0, 3000, 0.7, True, 97)
    ks = [4, 8, 1, 6]
    ctx0 = [30, 200, 0, 77]
    steps = 3
    B = len(ks)
    # a cache with room for every step's drafts
    case = wl.make_case(w, device=DEV, ctx=[c + steps * max(ks) for c in ctx0], k=ks)
    bt = case["block_table"]
    kv = tva.PagedKV(case["k_pool"], case["v_pool"], bt)
    state = torch.tensor([[c, c, c] for c in ctx0], dtype=torch.int32, device=DEV)
    ctx = torch.tensor(ctx0, dtype=torch.int32, device=DEV)
    cu = case["cu_q"]
    host_len = list(ctx0)
    max_len = max(ctx0) + steps * max(ks) + max(ks)
    for s in range(steps):
        say(f"kvmu loop step {s}")
        step = wl.make_case(w, device=DEV, ctx=host_len, k=ks, seed_offset=s + 1)
        batch = tva.Batch(ctx, cu, total_q=sum(ks), max_q=max(ks), max_len=max_len)
        tva.kvmu_apply(state, tva.KVMU_SPECULATE, torch.tensor(ks, dtype=torch.int32, device=DEV))
        tva.kv_append(batch, step["k_new"], step["v_new"], kv)
        out = tva.spec_verify_attn(batch, step["q"], kv, out_dtype=torch.float32)
        ids, n, nxt = tva.accept_prefix(batch, step["logits"], step["draft_ids"])
        tva.kvmu_apply(state, tva.KVMU_PREFIX, n, ctx_lens=ctx)
        torch.cuda.synchronize()
        # oracle on the same inputs: attention over the cache as it is now
        ref = oracle.spec_verify_attn(np_(step["q"]), np_(kv.k), np_(kv.v), np_(bt),
                                      np.array(host_len), np_(cu), 1.0 / math.sqrt(w.d))
        assert_close(out, ref, "bf16")
        _, rn, _ = oracle.accept_prefix(np_(step["logits"]), np_(step["draft_ids"]), np_(cu))
        assert np.array_equal(np_(n), rn)
        host_len = [h + int(x) for h, x in zip(host_len, rn)]
        assert np_(ctx).tolist() == host_len
        assert np_(state).tolist() == [[h, h, h] for h in host_len]
