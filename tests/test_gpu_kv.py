"""GPU parity of sva_kv_quant_int8 and sva_kv_append against the oracle, bit-exact
(INT8 codes, fp16 scales and stored cache bytes)."""
import numpy as np
import pytest
import torch

import oracle
import token_verify_attention_amd as tva
from token_verify_attention_amd import workloads as wl
from gpu_helpers import batch_of, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rows(n, d, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn((n, d), generator=g, device=DEV)
    mags = 10.0 ** torch.randint(-6, 6, (n, 1), generator=g, device=DEV).float()
    x = x * mags
    x[0] = 0.0                                              # zero row
    x[1, :] = 0.0
    x[1, :9] = torch.tensor([31.75, 0.125, 0.375, 0.625, -0.125, -0.375, -0.625,
                             0.12500001, 0.37499997])       # half-way ties
    x[2, :] = 1e-9                                          # fp16 scale underflows to 0
    x[3, :] = torch.linspace(-3e6, 3e6, d)                  # large magnitudes
    return x


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quant_bit_exact(d, src):
    say(f"quant d={d} src={src}")
    x = _rows(4096 + 3, d, d)
    if src == "bf16":
        x = x.to(torch.bfloat16)
    codes, scales = tva.kv_quant_int8(x)
    torch.cuda.synchronize()
    rc, rs = oracle.kv_quant_int8(np_(x))
    assert np.array_equal(np_(codes), rc)
    assert np.array_equal(np_(scales).view(np.uint16), rs.view(np.uint16))


def test_quant_full_cache_fill_sampled():
    """The 70B-shaped INT8 cache fill: every row of a random sample of pages."""
    w = wl.WORKLOADS["gqa70b_int8"]
    case = wl.make_case(w, device=DEV, with_logits=False)
    codes, scales = tva.kv_quant_int8(case["k_pool"])
    torch.cuda.synchronize()
    P = case["k_pool"].shape[0]
    pages = np.random.default_rng(1).choice(P, size=min(P, 512), replace=False)
    src = np_(case["k_pool"][torch.as_tensor(pages, device=DEV)])
    rc, rs = oracle.kv_quant_int8(src.reshape(-1, w.d))
    assert np.array_equal(np_(codes[torch.as_tensor(pages, device=DEV)]).reshape(-1, w.d), rc)
    got_s = np_(scales[torch.as_tensor(pages, device=DEV)]).reshape(-1)
    assert np.array_equal(got_s.view(np.uint16), rs.view(np.uint16))


def _pool_like(case, kvd):
    if kvd == "int8":
        P, H, _, d = case["k_pool"].shape
        z = lambda: torch.zeros((P, H, 16, d), dtype=torch.int8, device=DEV)
        s = lambda: torch.zeros((P, H, 16), dtype=torch.float16, device=DEV)
        return tva.PagedKV(z(), z(), case["block_table"], s(), s())
    dt = torch.float32 if kvd == "f32" else torch.bfloat16
    return tva.PagedKV(torch.zeros_like(case["k_pool"], dtype=dt),
                       torch.zeros_like(case["v_pool"], dtype=dt), case["block_table"])


@pytest.mark.parametrize("kvd", ["f32", "bf16", "int8"])
@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_append_bit_exact(kvd, src, d):
    say(f"append kv={kvd} src={src} d={d}")
    w = wl.Workload("app", 1, 8, 4, d, 0, 1, "f32", "f32", 1.0, None, None, True, 70 + d)
    case = wl.make_case(w, device=DEV, ctx=[0, 15, 16, 33, 200], k=[3, 1, 8, 0, 5],
                        with_logits=False)
    kn, vn = case["k_new"], case["v_new"]
    if src == "bf16":
        kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    kv = _pool_like(case, kvd)
    tva.kv_append(batch_of(case), kn, vn, kv)
    torch.cuda.synchronize()
    bt, ctx, cu = np_(case["block_table"]), np_(case["ctx_lens"]), np_(case["cu_q"])
    if kvd == "int8":
        zc = np.zeros(kv.k.shape, np.int8)
        zs = np.zeros(kv.k_scale.shape, np.float16)
        rk, rv, rks, rvs = oracle.kv_append(np_(kn), np_(vn), zc, zc, bt, ctx, cu, "int8", zs, zs)
        assert np.array_equal(np_(kv.k), rk) and np.array_equal(np_(kv.v), rv)
        assert np.array_equal(np_(kv.k_scale).view(np.uint16), rks.view(np.uint16))
        assert np.array_equal(np_(kv.v_scale).view(np.uint16), rvs.view(np.uint16))
    else:
        z = np.zeros(kv.k.shape)
        rk, rv, _, _ = oracle.kv_append(np_(kn), np_(vn), z, z, bt, ctx, cu, kvd)
        assert np.array_equal(np_(kv.k).astype(np.float64), rk)
        assert np.array_equal(np_(kv.v).astype(np.float64), rv)


def test_append_full_size_8b_gqa():
    """The 8B-GQA workload's append: written rows exact, the rest untouched."""
    w = wl.WORKLOADS["gqa8b"]
    case = wl.make_case(w, device=DEV, with_logits=False)
    before_k = case["k_pool"].clone()
    kv = tva.PagedKV(case["k_pool"], case["v_pool"], case["block_table"])
    tva.kv_append(batch_of(case), case["k_new"], case["v_new"], kv)
    torch.cuda.synchronize()
    bt, ctx, cu = np_(case["block_table"]), np_(case["ctx_lens"]), np_(case["cu_q"])
    written = torch.zeros(case["k_pool"].shape[:3], dtype=torch.bool)
    for b in range(w.B):
        for i in range(int(cu[b + 1] - cu[b])):
            pos = int(ctx[b]) + i
            pg, sl = int(bt[b, pos // 16]), pos % 16
            assert torch.equal(case["k_pool"][pg, :, sl], case["k_new"][int(cu[b]) + i])
            assert torch.equal(case["v_pool"][pg, :, sl], case["v_new"][int(cu[b]) + i])
            written[pg, :, sl] = True
    keep = ~written.to(DEV)
    assert torch.equal(case["k_pool"][keep], before_k[keep])
