"""Shared pieces of the GPU parity tests: marshal a synthetic case into the
binding's objects and the oracle's numpy arrays, and the tolerance rules.

Tolerances (max |err| over the compared outputs):
  bf16 cache, bf16 output        1e-2 * max|ref| + 1e-3
  INT8 cache vs unquantised ref  3e-2 * max|ref| + 1e-3
  INT8 cache vs dequantised ref  1e-2 * max|ref| + 1e-3
  fp32 cache, fp32 output        1e-4 * max|ref| + 1e-5
The pages state no tolerance for fp32; the last one is derived from the
arithmetic: fp32 dot products of d <= 128 terms err by about
sqrt(d) * 2^-24 * sum|q_c K_c| * scale (~1e-6 for N(0,1) data), v_exp_f32 adds
about one ulp, and the weights and P.V sums stay fp32, so outputs carry a
relative error near 1e-6; the bar sits two orders of magnitude above that and
far below the effect of a structural mistake (a dropped key moves outputs by
~1e-2).
"""
import math
import sys

import numpy as np
import torch

import oracle
import token_verify_attention_amd as tva
from token_verify_attention_amd import workloads as wl

TOL = {"bf16": (1e-2, 1e-3), "int8": (3e-2, 1e-3), "int8_deq": (1e-2, 1e-3), "f32": (1e-4, 1e-5)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def batch_of(case):
    return tva.Batch(case["ctx_lens"], case["cu_q"], total_q=case["T"], max_q=case["max_q"],
                     max_len=case["max_len"])


def quantise_pool(pool):
    """INT8 codes + fp16 scales of a [P, Hkv, 16, d] fp32 pool, on the GPU."""
    return tva.kv_quant_int8(pool)


def paged_kv(case, kv_dtype=None):
    """The binding's PagedKV for the case; INT8 pools are quantised on the GPU."""
    kv_dtype = kv_dtype or case["workload"].kv_dtype
    if kv_dtype == "int8":
        kc, ks = quantise_pool(case["k_pool"])
        vc, vs = quantise_pool(case["v_pool"])
        return tva.PagedKV(kc, vc, case["block_table"], ks, vs)
    return tva.PagedKV(case["k_pool"], case["v_pool"], case["block_table"])


def np_(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def oracle_attn(case, kv_dtype=None, quantised=True, select=None, q=None):
    """Oracle output for the case.  INT8: quantised=True quantises the fp32
    pool with the oracle's own quantiser; False uses the unquantised values."""
    w = case["workload"]
    kv_dtype = kv_dtype or w.kv_dtype
    qn = np_(case["q"] if q is None else q)
    kp, vp = np_(case["k_pool"]), np_(case["v_pool"])
    args = dict(select=select)
    if kv_dtype == "int8" and quantised:
        P, H = kp.shape[:2]
        kc, ks = oracle.kv_quant_int8(kp.reshape(-1, w.d))
        vc, vs = oracle.kv_quant_int8(vp.reshape(-1, w.d))
        kp, vp = kc.reshape(kp.shape), vc.reshape(vp.shape)
        args.update(k_scale=ks.reshape(P, H, 16), v_scale=vs.reshape(P, H, 16))
    return oracle.spec_verify_attn(qn, kp, vp, np_(case["block_table"]), np_(case["ctx_lens"]),
                                   np_(case["cu_q"]), 1.0 / math.sqrt(w.d), **args)


def assert_close(got, ref, kind, rows=None):
    """max |got - ref| <= rtol * max|ref| + atol over the rows compared."""
    got = np_(got).astype(np.float64) if isinstance(got, torch.Tensor) else got
    if rows is not None:
        got, ref = got[rows], ref[rows]
    mask = ~np.isnan(ref)
    assert mask.any()
    assert np.isfinite(got[mask]).all(), "non-finite output"
    err = np.abs(got[mask] - ref[mask]).max()
    rtol, atol = TOL[kind]
    bound = rtol * np.abs(ref[mask]).max() + atol
    assert err <= bound, f"{kind}: max err {err:.3e} > bound {bound:.3e}"
    return err, bound


def rows_of_pairs(case, pairs):
    """Flat (row, head) mask of the outputs that belong to the given (b, g)."""
    w = case["workload"]
    G = w.Hq // w.Hkv
    cu = case["cu_q"].cpu().numpy()
    m = np.zeros((case["T"], w.Hq), bool)
    for b, g in pairs:
        m[cu[b]:cu[b + 1], g * G:(g + 1) * G] = True
    return m
