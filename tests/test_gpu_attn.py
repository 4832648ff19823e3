"""GPU parity of sva_spec_verify_attn against the fp64 oracle (through the C ABI).

Small cases span several pages, ragged tails (S = 0, 1, 15, 16, 17, ...), k = 1..16,
GQA groups 1..8, d = 64 / 128, fp32 / bf16 / INT8 caches and both inner paths,
grid sizes that force pairs to be split over workgroups (the cross-workgroup
merge), and pairs whose kv head's query heads are split over workgroups (to
fit one 32-row pass, or because the pairs are few) as well as unsplit ones.  Full-size workloads are checked on every (sequence, kv-head) pair, through
the call and launch configuration the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import token_verify_attention_amd as tva
from token_verify_attention_amd import workloads as wl
from gpu_helpers import (assert_close, batch_of, np_, oracle_attn, paged_kv, rows_of_pairs,
                         say)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

W = wl.Workload


def _wk(name, Hq, Hkv, d, kv, q, sigma=1.0, ident=50):
    return W(name, 1, Hq, Hkv, d, 0, 1, kv, q, sigma, None, None, False, ident)


SMALL = [
    # workload, ctx lengths, draft counts
    (_wk("mha-bf16-d128", 8, 8, 128, "bf16", "bf16", ident=51), [0, 1, 15, 16, 17, 100, 300], [4, 1, 3, 4, 2, 4, 4]),
    (_wk("gqa4-bf16-d128", 16, 4, 128, "bf16", "bf16", ident=52), [33, 250, 5, 64, 0], [8, 5, 1, 4, 3]),
    (_wk("gqa8-int8-d128", 32, 4, 128, "int8", "bf16", 0.5, ident=53), [200, 17, 511, 3], [4, 3, 2, 1]),
    (_wk("tiny-f32-d64", 4, 4, 64, "f32", "f32", ident=54), [128, 40, 0], [4, 3, 2]),
    (_wk("gqa2-bf16-d64", 8, 4, 64, "bf16", "bf16", ident=55), [70, 1, 31], [7, 8, 2]),
    (_wk("gqa4-int8-d64", 16, 4, 64, "int8", "f32", 0.5, ident=56), [90, 16, 47], [5, 4, 8]),
    (_wk("rows128-bf16", 16, 2, 128, "bf16", "bf16", ident=57), [50, 3], [16, 16]),
    (_wk("gqa2-f32-d128", 8, 4, 128, "f32", "bf16", ident=65), [0, 300, 17, 64], [3, 4, 8, 1]),
    # 36 (sequence, kv head) pairs of 32 query rows, more pairs than the
    # planner splits into query-head halves on a 256-CU part: unsplit pairs
    # at small sizes; and 36 pairs of 64 rows, split in two to fit one pass
    (_wk("gqa4-36pairs-bf16", 16, 4, 128, "bf16", "bf16", ident=88),
     [0, 1, 15, 16, 17, 100, 300, 64, 31], [4, 1, 3, 4, 2, 8, 4, 5, 1]),
    (_wk("gqa4-36pairs-int8", 16, 4, 128, "int8", "bf16", 0.5, ident=89),
     [5, 40, 200, 17, 0, 96, 33, 300, 63], [2, 4, 1, 8, 3, 4, 6, 2, 4]),
    (_wk("gqa8-36pairs-64rows", 32, 4, 128, "bf16", "bf16", ident=85),
     [9, 70, 0, 33, 130, 16, 250, 47, 5], [8, 3, 5, 8, 1, 6, 8, 2, 7]),
]


def _case(w, ctx, ks, **kw):
    return wl.make_case(w, device=DEV, ctx=ctx, k=ks, with_logits=False, **kw)


def _kind(w):
    return {"bf16": "bf16", "int8": "int8", "f32": "f32"}[w.kv_dtype]


def _check(case, out, kind_dtype=None):
    w = case["workload"]
    kind = kind_dtype or w.kv_dtype
    if kind == "int8":
        ref_q = oracle_attn(case, quantised=True)
        ref_u = oracle_attn(case, quantised=False)
        assert_close(out, ref_q, "int8_deq")
        return assert_close(out, ref_u, "int8")
    ref = oracle_attn(case)
    # the fp32 bound needs an fp32 cache and an fp32 output: a bf16 output
    # rounds each value to 8 significant bits whatever the cache holds
    tight = kind == "f32" and out.dtype == torch.float32
    return assert_close(out, ref, "f32" if tight else "bf16")


@pytest.mark.parametrize("path", [0, 1, 2], ids=["auto", "valu", "mfma"])
@pytest.mark.parametrize("spec", SMALL, ids=[s[0].name for s in SMALL])
def test_small_cases(spec, path):
    w, ctx, ks = spec
    say(f"attn small {w.name} path={path}")
    case = _case(w, ctx, ks)
    kv = paged_kv(case)
    out = tva.spec_verify_attn(batch_of(case), case["q"], kv, path=path)
    torch.cuda.synchronize()
    _check(case, out)


@pytest.mark.parametrize("nwg", [1, 2, 3, 7, 64, 300])
def test_pairs_split_over_workgroups(nwg):
    w = _wk("split-gqa4", 16, 4, 128, "bf16", "bf16", ident=58)
    say(f"attn split W={nwg}")
    case = _case(w, [700, 33, 1, 260], [4, 8, 2, 3])
    kv = paged_kv(case)
    out = tva.spec_verify_attn(batch_of(case), case["q"], kv, num_workgroups=nwg)
    torch.cuda.synchronize()
    _check(case, out)


def test_fp32_output_from_bf16_cache():
    w = _wk("f32out", 16, 4, 128, "bf16", "bf16", ident=59)
    case = _case(w, [300, 45], [4, 6])
    out = tva.spec_verify_attn(batch_of(case), case["q"], paged_kv(case), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    _check(case, out)


@pytest.mark.parametrize("path", [0, 1], ids=["auto", "valu"])
def test_fp32_cache_d128_fp32_output(path):
    """An fp32 cache at d = 128 read with bf16 queries, written as fp32: held
    to the fp32 bound, on pairs that span several pages and a ragged tail."""
    w = _wk("f32out-d128", 8, 4, 128, "f32", "bf16", ident=66)
    case = _case(w, [0, 300, 17, 64, 511], [3, 4, 8, 1, 6])
    say(f"attn f32 cache d128 f32 out path={path}")
    out = tva.spec_verify_attn(batch_of(case), case["q"], paged_kv(case),
                               out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    _check(case, out)


@pytest.mark.parametrize("kvd", ["bf16", "int8", "f32"])
def test_poisoned_garbage_slots_and_pages_never_leak(kvd):
    """NaN in every slot past S_b + k_b and in unreferenced pages; -1 in
    unused block-table entries.  Outputs equal the unpoisoned run bitwise."""
    w = _wk(f"poison-{kvd}", 16, 4, 128, kvd, "bf16", 0.5 if kvd == "int8" else 1.0, ident=60)
    ctx, ks = [37, 250, 1, 16], [3, 8, 2, 4]
    clean = _case(w, ctx, ks, extra_pages=5)
    dirty = _case(w, ctx, ks, extra_pages=5, poison=True)
    kv_c = paged_kv(clean)
    if kvd == "int8":
        kv_d = paged_kv(clean)              # same codes; poison the scales instead
        for t in (kv_d.k_scale, kv_d.v_scale):
            pb = dirty["block_table"].cpu()
            for b, (c, k) in enumerate(zip(ctx, ks)):
                used = c + k
                if used % 16:
                    t[int(pb[b, (used - 1) // 16]), :, used % 16:] = float("nan")
    else:
        kv_d = paged_kv(dirty)
    a = tva.spec_verify_attn(batch_of(clean), clean["q"], kv_c)
    b = tva.spec_verify_attn(batch_of(dirty), dirty["q"], kv_d)
    torch.cuda.synchronize()
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a, b)


@pytest.mark.parametrize("kvd", ["bf16", "int8"])
def test_later_drafts_do_not_change_earlier_queries(kvd):
    w = _wk(f"prefix-{kvd}", 32, 4, 128, kvd, "bf16", ident=61)
    ctx, ks = [77, 300], [6, 5]
    case = _case(w, ctx, ks)
    base = tva.spec_verify_attn(batch_of(case), case["q"], paged_kv(case)).clone()
    bt = case["block_table"].cpu()
    cu = case["cu_q"].cpu()
    for b in range(2):
        for j in range(ks[b] - 1):
            pert = dict(case)
            kp, vp = case["k_pool"].clone(), case["v_pool"].clone()
            for jj in range(j + 1, ks[b]):
                pos = ctx[b] + jj
                pg = int(bt[b, pos // 16])
                kp[pg, :, pos % 16] += 3.0
                vp[pg, :, pos % 16] = 50.0
            pert["k_pool"], pert["v_pool"] = kp, vp
            got = tva.spec_verify_attn(batch_of(pert), case["q"], paged_kv(pert))
            rows = slice(int(cu[b]), int(cu[b]) + j + 1)
            assert torch.equal(got[rows], base[rows]), (b, j)


def test_deterministic_across_runs():
    w = _wk("det", 32, 8, 128, "bf16", "bf16", ident=62)
    case = _case(w, [1000, 17, 400], [4, 8, 2])
    kv = paged_kv(case)
    outs = [tva.spec_verify_attn(batch_of(case), case["q"], kv, num_workgroups=5).clone()
            for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


def test_zero_drafts():
    w = _wk("zero", 8, 4, 128, "bf16", "bf16", ident=63)
    case = _case(w, [30, 50, 70], [0, 3, 0])
    out = tva.spec_verify_attn(batch_of(case), case["q"], paged_kv(case))
    torch.cuda.synchronize()
    _check(case, out)
    empty = _case(w, [30, 50], [0, 0])
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=DEV)
    out = tva.spec_verify_attn(batch_of(empty), q, paged_kv(empty))
    assert out.shape == (0, 8, 128)


def _own_cache(case):
    """A cache of the case's own (an INT8 cache is quantised afresh; float
    pools are cloned), so two calls never write the same memory."""
    if case["workload"].kv_dtype == "int8":
        return paged_kv(case)
    return tva.PagedKV(case["k_pool"].clone(), case["v_pool"].clone(), case["block_table"])


def _cache_bits(kv):
    parts = [kv.k.view(torch.int8), kv.v.view(torch.int8)]
    if kv.k_scale is not None:
        parts += [kv.k_scale.view(torch.int16), kv.v_scale.view(torch.int16)]
    return parts


@pytest.mark.parametrize("name", ["tiny", "mha7b", "gqa8b", "gqa70b_int8", "gqa70b_int8_tp8",
                                  "ragged"])
def test_full_size_workloads_every_pair(name):
    """The call the benchmark times -- sva_spec_verify_attn_append: the k_b new
    rows appended and the drafts verified in one launch, default launch
    configuration -- at the workload's full size, against the oracle's append
    then attention on every (sequence, kv-head) pair; the same step as two
    calls (sva_kv_append, then sva_spec_verify_attn) gives the same bits and
    the same cache."""
    w = wl.WORKLOADS[name]
    say(f"attn full-size {name}: generating")
    case = wl.make_case(w, device=DEV, with_logits=False)
    kp, vp = np_(case["k_pool"]), np_(case["v_pool"])        # before the GPU append
    batch = batch_of(case)
    kv_fused, kv_two = _own_cache(case), _own_cache(case)
    out = tva.spec_verify_attn_append(batch, case["q"], kv_fused, case["k_new"], case["v_new"])
    tva.kv_append(batch, case["k_new"], case["v_new"], kv_two)
    out_two = tva.spec_verify_attn(batch, case["q"], kv_two)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int8), out_two.view(torch.int8))
    for a, b in zip(_cache_bits(kv_fused), _cache_bits(kv_two)):
        assert torch.equal(a, b)
    del kv_two, out_two
    say(f"attn full-size {name}: kernels done, oracle on every pair")
    ctx, cu, bt = np_(case["ctx_lens"]), np_(case["cu_q"]), np_(case["block_table"])
    kn, vn = np_(case["k_new"]), np_(case["v_new"])
    scale = 1.0 / math.sqrt(w.d)
    qn = np_(case["q"])
    if w.kv_dtype == "int8":
        P, H = kp.shape[:2]
        kc, ksc = oracle.kv_quant_int8(kp.reshape(-1, w.d))
        vc, vsc = oracle.kv_quant_int8(vp.reshape(-1, w.d))
        kc, vc, ksc, vsc = oracle.kv_append(kn, vn, kc.reshape(kp.shape), vc.reshape(vp.shape),
                                            bt, ctx, cu, "int8", ksc.reshape(P, H, 16),
                                            vsc.reshape(P, H, 16))
        # the cache the GPU wrote: codes and scales bit-exact
        assert np.array_equal(np_(kv_fused.k), kc) and np.array_equal(np_(kv_fused.v), vc)
        assert np.array_equal(np_(kv_fused.k_scale).view(np.uint16), ksc.view(np.uint16))
        assert np.array_equal(np_(kv_fused.v_scale).view(np.uint16), vsc.view(np.uint16))
        ref_q = oracle.spec_verify_attn(qn, kc, vc, bt, ctx, cu, scale, k_scale=ksc,
                                        v_scale=vsc)
        assert_close(out, ref_q, "int8_deq")
        del kc, vc
        kp, vp, _, _ = oracle.kv_append(kn, vn, kp, vp, bt, ctx, cu, "f32")
        ref_u = oracle.spec_verify_attn(qn, kp, vp, bt, ctx, cu, scale)
        assert_close(out, ref_u, "int8")
    else:
        kp, vp, _, _ = oracle.kv_append(kn, vn, kp, vp, bt, ctx, cu, w.kv_dtype)
        ref = oracle.spec_verify_attn(qn, kp, vp, bt, ctx, cu, scale)
        assert_close(out, ref, "f32" if w.kv_dtype == "f32" else "bf16")
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("variant", ["fused", "two_pass", "valu"])
def test_one_workspace_serves_calls_of_any_grid_size(variant):
    """Regression: partial slots of a call with a small grid must not land on
    the completion counters of a later call with a larger grid, and every call
    leaves the counters zero -- on the fused merge (at most 32 query rows per
    pair), the per-pass merge (64 rows: two passes) and the VALU path."""
    ks = [16, 9, 2, 12] if variant == "two_pass" else [4, 8, 2, 3]
    path = tva.PATH_VALU if variant == "valu" else tva.PATH_AUTO
    w = _wk("ws-reuse", 32, 8, 128, "bf16", "bf16", ident=64)
    case = _case(w, [2000, 700, 33, 1500], ks)
    kv = paged_kv(case)
    batch = batch_of(case)
    nmax = max(tva.verify_workspace_bytes(batch, kv, w.Hq, path=path, num_workgroups=n)
               for n in (3, 5, 17, 256, 1024))
    ws = torch.zeros(nmax, dtype=torch.uint8, device=DEV)
    ref = oracle_attn(case)
    for n in (5, 256, 3, 1024, 17, 0):
        say(f"workspace reuse {variant} nwg={n}")
        out = tva.spec_verify_attn(batch, case["q"], kv, workspace=ws, num_workgroups=n,
                                   path=path)
        torch.cuda.synchronize()
        assert_close(out, ref, "bf16")
        assert int(ws[:32768].count_nonzero()) == 0, n


@pytest.mark.parametrize("name,nwg", [("gqa70b_int8", 0), ("gqa70b_int8_tp8", 0), ("gqa8b", 600)])
def test_split_pairs_are_bit_reproducible(name, nwg):
    """Pairs split over several workgroups are merged in segment order by
    whichever workgroup arrives last; which one that is varies from run to
    run, the result must not: repeated calls give identical bits."""
    w = wl.WORKLOADS[name]
    case = wl.make_case(w, device=DEV, with_logits=False)
    batch = batch_of(case)
    kv = paged_kv(case)
    say(f"attn reproducibility {name} nwg={nwg}")
    outs = [tva.spec_verify_attn(batch, case["q"], kv, num_workgroups=nwg) for _ in range(6)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert torch.isfinite(outs[0].float()).all()


@pytest.mark.parametrize("kvd,nwg", [("bf16", 0), ("bf16", 600), ("int8", 300)])
def test_long_context_few_pairs_many_segments(kvd, nwg):
    """One long sequence over two kv heads: each pair is split over tens to
    hundreds of workgroups, so the last one folds many partials (more than
    one table's worth at 600 workgroups)."""
    w = _wk(f"long-ctx-{kvd}", 8, 2, 128, kvd, "bf16", 0.5 if kvd == "int8" else 1.0, ident=70)
    case = _case(w, [60000], [4])
    batch = batch_of(case)
    kv = paged_kv(case)
    say(f"attn long context {kvd} nwg={nwg}")
    outs = [tva.spec_verify_attn(batch, case["q"], kv, num_workgroups=nwg) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    _check(case, outs[0])


# G = 8, up to 4 drafts (32 query rows per pair) and 16 (sequence, kv head)
# pairs: few enough pairs that each kv head's query heads are split into two
# halves streamed (and merged) apart, so the unit that gives up is half a
# pair.  G = 3 cannot be halved: the unit is the whole pair.
GIVE_UP = [(_wk("giveup", 32, 4, 128, "bf16", "bf16", ident=71), 2),
           (_wk("giveup-g3", 12, 4, 128, "bf16", "bf16", ident=87), 1)]


@pytest.mark.parametrize("spec", GIVE_UP, ids=[s[0].name for s in GIVE_UP])
def test_wait_that_gives_up_writes_nan_and_leaves_the_workspace_reusable(spec):
    """Forced from the host: with no poll allowed, the workgroup that finishes
    each split pair gives up at once instead of waiting for the others'
    partials.  Its rows must come out NaN (never a fold of partials that may
    be missing) for every query head of the unit that gave up, the status
    word must say so, and once every workgroup is done the counters must be
    back at zero, so the same workspace then serves an ordinary call.  Every
    kernel exits normally."""
    w, parts = spec
    case = _case(w, [3000, 40, 1200, 700], [4, 2, 3, 4])
    batch = batch_of(case)
    kv = paged_kv(case)
    ws = torch.zeros(tva.verify_workspace_bytes(batch, kv, w.Hq, num_workgroups=24),
                     dtype=torch.uint8, device=DEV)
    say("attn forced give-up")
    bad = tva.spec_verify_attn(batch, case["q"], kv, workspace=ws, num_workgroups=24,
                               wait_polls=-1)
    torch.cuda.synchronize()
    assert int(ws[:tva.STATUS_OFFSET].count_nonzero()) == 0     # counters back at zero
    assert tva.verify_status(ws) == 1                           # read and cleared
    assert tva.verify_status(ws) == 0
    ref = oracle_attn(case)
    got = np_(bad).astype(np.float64)
    U = w.Hq // w.Hkv // parts                     # query heads per unit
    cu = np_(case["cu_q"])
    nan_units = 0
    for b in range(case["B"]):
        for u in range(w.Hkv * parts):
            blk = got[cu[b]:cu[b + 1], u * U:(u + 1) * U]
            if np.isnan(blk).any():
                assert np.isnan(blk).all(), (b, u)              # the whole unit, never a part
                nan_units += 1
            else:
                assert_close(blk, ref[cu[b]:cu[b + 1], u * U:(u + 1) * U], "bf16")
    assert nan_units > 0
    good = tva.spec_verify_attn(batch, case["q"], kv, workspace=ws, num_workgroups=24)
    torch.cuda.synchronize()
    assert tva.verify_status(ws) == 0
    assert_close(good, ref, "bf16")


def test_calls_on_a_side_stream():
    """Outputs and workspaces the binding allocates for a call on another
    stream are allocated on that stream; results equal the default stream's."""
    w = W("side-stream", 1, 16, 4, 128, 0, 1, "bf16", "bf16", 1.0, 4099, 0.7, False, 72)
    case = wl.make_case(w, device=DEV, ctx=[500, 70, 2000], k=[4, 3, 8])
    batch = batch_of(case)
    kv = paged_kv(case)
    ref = tva.spec_verify_attn(batch, case["q"], kv)
    ref_acc = tva.accept_prefix(batch, case["logits"], case["draft_ids"])
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=DEV)
    for _ in range(3):
        out = tva.spec_verify_attn(batch, case["q"], kv, stream=s, num_workgroups=9)
        acc = tva.accept_prefix(batch, case["logits"], case["draft_ids"], stream=s)
    s.synchronize()
    keys = [k for k in tva._ws_cache if k[1] == s.cuda_stream]
    assert keys, "no workspace of its own for the side stream"
    assert_close(out, oracle_attn(case), "bf16")
    assert_close(ref, oracle_attn(case), "bf16")
    for a, b in zip(acc, ref_acc):
        assert torch.equal(a, b)


@pytest.mark.parametrize("vmode", ["small", "mixed", "large"])
def test_int8_value_rows_of_other_magnitudes(vmode):
    """INT8 caches at S = 8192 with V rows far from N(0, 0.5): all small
    (N(0, 1e-2): scales near 2e-4, so most weight x scale products are fp16
    subnormals), magnitudes spread over four decades row by row, and large
    rows (scales near 200, the products' upper range).  Both bars hold and no
    output is non-finite."""
    w = _wk(f"int8-v-{vmode}", 32, 4, 128, "int8", "bf16", 0.5, ident=73)
    case = _case(w, [8192, 3000], [4, 3])
    v = case["v_pool"]
    g = torch.Generator(device=DEV)
    g.manual_seed(7300)
    if vmode == "small":
        v.mul_(0.02)
    elif vmode == "mixed":
        u = torch.rand(v.shape[:3], generator=g, device=DEV) * -4.0
        v.mul_(torch.pow(10.0, u).unsqueeze(-1))
    else:
        v.mul_(12000.0 / v.abs().amax())
    say(f"attn int8 V magnitudes {vmode}")
    out = tva.spec_verify_attn(batch_of(case), case["q"], paged_kv(case))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ref_q = oracle_attn(case, quantised=True)
    err, bound = assert_close(out, ref_q, "int8_deq")
    rel = err / np.abs(ref_q).max()
    say(f"  max err {err:.3e}, {rel:.2e} of max|ref| (bound {bound:.3e})")
    assert_close(out, oracle_attn(case, quantised=False), "int8")


@pytest.mark.parametrize("kvd,path", [("bf16", 0), ("bf16", 1), ("int8", 0), ("f32", 0)])
@pytest.mark.parametrize("scale", [-0.05, 0.3, 1e-3])
def test_softmax_scales_other_than_the_default(kvd, path, scale):
    """Any finite non-zero softmax scale, negative included (the bf16 MFMA
    path moves a negative scale's sign into Q), on the split kernel and on
    the row-block kernel (40 drafts)."""
    w = _wk(f"scale-{kvd}", 16, 4, 128 if kvd != "f32" else 64, kvd,
            "bf16" if kvd != "f32" else "f32", 0.5 if kvd == "int8" else 1.0, ident=74)
    ks = [4, 9, 2] if kvd == "f32" or path == 1 else [4, 40, 2]
    case = _case(w, [300, 70, 1000], ks)
    say(f"attn scale={scale} {kvd} path={path}")
    out = tva.spec_verify_attn(batch_of(case), case["q"], paged_kv(case), softmax_scale=scale,
                               path=path)
    torch.cuda.synchronize()
    qn = np_(case["q"])
    kp, vp = np_(case["k_pool"]), np_(case["v_pool"])
    bt, ctx, cu = np_(case["block_table"]), np_(case["ctx_lens"]), np_(case["cu_q"])
    ref = oracle.spec_verify_attn(qn, kp, vp, bt, ctx, cu, scale)
    assert_close(out, ref, {"int8": "int8", "f32": "f32", "bf16": "bf16"}[kvd])
