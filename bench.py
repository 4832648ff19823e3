"""Benchmark of the speculative-verification hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic batch:
  spec_verify_attn_append (the k new K/V rows of every sequence written into
  the cache -- INT8 caches quantise on write -- and the drafts verified, one
  launch) -> accept_prefix (argmax over the vocabulary and the longest
  accepted prefix).  Token-tree workloads (--workload tree8b) run
  tree_masks -> the same call with the tree masks -> accept_tree_commit (the
  tree walk and the commit of the accepted branch, one launch after the
  argmax); --workload ragged_sampled replaces greedy acceptance by
  stochastic acceptance (rejection sampling over target and drafter logits);
  --workload prm7b_step verifies long speculated steps (128 drafts per
  sequence, the attention shape of a 7B process reward model): kv_append ->
  verification attention, whose roofline is MFMA throughput (the reward
  model's threshold is not part of this path).
Default workload: 7B-MHA shape, B=8, Hq=Hkv=32, d=128, S=2048, k=4, bf16 paged
KV (16-token pages, random page permutation).  That shape names no vocabulary;
acceptance runs over fp32 logits [B*(k+1), 128256] with drafts agreeing with
the target argmax with probability 0.8 (the ragged serving batch's vocabulary
and agreement rate).

Prints ONE JSON line.  `value` is verified draft tokens per second for whole
steps (inputs resident in HBM); `roofline` is the attention kernel's KV bytes
over its own average launch time against 8 TB/s; `cpu_baseline` is the fp64
oracle on the host.  The attention kernel's average launch time comes from
the same number of back-to-back launches of the attention call alone
(sva_spec_verify_attn, no append) after the timed steps, between one pair of
HIP events on its stream; `roofline.traffic` is HBM traffic from committed rocprofv3
counter readings (null when they no longer match the kernel's sources).
"""
import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np
import torch

METRIC = "verify-attn KV HBM GB/s (% of peak) and verified draft tokens/sec, 1 GPU"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes(w, ctx, ks):
    """Algorithmic KV bytes of one verify-attn launch: K and V rows 0..S_b+k_b-1
    of every kv head, plus the fp16 scale of every INT8 row."""
    elem = {"f32": 4, "bf16": 2, "int8": 1}[w.kv_dtype]
    per_row = w.d * elem + (2 if w.kv_dtype == "int8" else 0)
    rows = sum(c + k for c, k in zip(ctx, ks))
    return 2 * w.Hkv * rows * per_row


def attn_flops(w, ctx, ks):
    """Algorithmic FLOPs of one verify-attn launch: per query row of draft i
    (G rows per draft and kv head), S_b + i + 1 visible keys, each costing a
    d-long dot product for the score and a d-long multiply-add into the
    output (2 FLOPs per multiply-add)."""
    G = w.Hq // w.Hkv
    total = 0
    for c, k in zip(ctx, ks):
        keys = k * (c + 1) + k * (k - 1) // 2          # sum over drafts of S + i + 1
        total += 4 * w.d * keys * G * w.Hkv
    return total


def other_bytes(w, ctx, ks, max_pages):
    qe = {"f32": 4, "bf16": 2}[w.q_dtype]
    T = sum(ks)
    return 2 * T * w.Hq * w.d * qe + 4 * len(ctx) * max_pages + 8 * len(ctx)


KERNEL_SOURCES = ("verify_attn.hip", "common.h", "launch.h", "kv_rows.h")


def kernel_source_hash():
    """sha256 over the attention kernel's sources, to tell whether stored
    counter readings still describe the kernel as built."""
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "token_verify_attention_amd",
                        "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(base, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, attn_ms):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    readings (each scaled by what the counter reads for a plain copy of known
    size), as a rate over this run's average launch time.  None when no
    reading exists for the workload or the kernel sources changed since."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"verify_attn_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    nbytes = float(kv["traffic_bytes_per_launch"])
    return {"bytes": nbytes, "gbps": nbytes / (attn_ms * 1e-3) / 1e9}


class Inputs:
    """One resident input set and the prepared calls of one step."""

    def __init__(self, tva, wl, w, seed_offset, dev):
        tree = w.name in wl.TREE_WORKLOADS
        long = w.name in wl.LONG_WORKLOADS
        self.case = case = wl.make_case(w, device=dev, seed_offset=seed_offset,
                                        with_logits=not (tree or long))
        if tree:
            case["parents"] = wl.make_tree(case["k_host"], device=dev, seed=w.ident + 97 * seed_offset)
            case.update(wl.make_tree_logits(w, case["k_host"], case["parents"], device=dev,
                                            seed_offset=seed_offset))
        self.batch = tva.Batch(case["ctx_lens"], case["cu_q"], total_q=case["T"],
                               max_q=case["max_q"], max_len=case["max_len"])
        if w.kv_dtype == "int8":
            kc, ks = tva.kv_quant_int8(case["k_pool"])
            vc, vs = tva.kv_quant_int8(case["v_pool"])
            self.kv = tva.PagedKV(kc, vc, case["block_table"], ks, vs)
        else:
            self.kv = tva.PagedKV(case["k_pool"], case["v_pool"], case["block_table"])
        self.out = torch.empty_like(case["q"])
        B = case["B"]
        self.ids = torch.empty(case["T"] + B, dtype=torch.int32, device=dev)
        self.alen = torch.empty(B, dtype=torch.int32, device=dev)
        self.nxt = torch.empty(B, dtype=torch.int32, device=dev)
        self.append = tva.prepare_kv_append(self.batch, case["k_new"], case["v_new"], self.kv)
        if tree:
            self.masks = torch.empty(case["T"], dtype=torch.int32, device=dev)
            self.path = torch.empty(case["T"], dtype=torch.int32, device=dev)
            self.tree_masks = tva.prepare_tree_masks(self.batch, case["parents"], self.masks)
            self.tree_masks()
            self.attn = tva.prepare_spec_verify_attn(self.batch, case["q"], self.kv, self.out,
                                                     draft_mask=self.masks)
            # the step appends and verifies in one call (one launch)
            fused = tva.prepare_spec_verify_attn_append(self.batch, case["q"], self.kv,
                                                        case["k_new"], case["v_new"], self.out,
                                                        draft_mask=self.masks)
            self.append = lambda stream=None: None
            self.accept = tva.prepare_accept_tree_commit(self.batch, case["logits"],
                                                         case["draft_ids"], case["parents"],
                                                         self.kv, self.ids, self.alen, self.nxt,
                                                         self.path)
            masks_call = self.tree_masks

            def step_attn(stream=None):
                masks_call(stream)
                fused(stream)
            self.step_attn = step_attn
        else:
            self.attn = tva.prepare_spec_verify_attn(self.batch, case["q"], self.kv, self.out)
            if long:
                self.accept = lambda stream=None: None
            elif w.name in wl.SAMPLED_WORKLOADS:
                case["draft_logits"] = wl.make_draft_logits(case["logits"], case["k_host"],
                                                            device=dev, seed=w.ident + seed_offset)
                case["u_accept"], case["u_sample"] = wl.make_uniforms(
                    case["T"], B, device=dev, seed=w.ident + seed_offset)
                self.accept = tva.prepare_accept_stochastic(
                    self.batch, case["logits"], case["draft_logits"], case["draft_ids"],
                    case["u_accept"], case["u_sample"], self.alen, self.nxt)
            else:
                self.accept = tva.prepare_accept_prefix(self.batch, case["logits"],
                                                        case["draft_ids"], self.ids, self.alen,
                                                        self.nxt)
            if long:
                # the row-block kernel appends in a launch of its own anyway
                self.step_attn = self.attn
            else:
                # the step appends and verifies in one call (one launch)
                self.step_attn = tva.prepare_spec_verify_attn_append(
                    self.batch, case["q"], self.kv, case["k_new"], case["v_new"], self.out)
                self.append = lambda stream=None: None


def copy_probe_gbps(dev, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy, the achievable-bandwidth reference."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def cpu_baseline(wl, w, dev, budget_s):
    """The fp64 oracle (as it stands) on a bounded sample of the same step:
    append + attention over (sequence, kv-head) pairs taken in order (cycling
    over the batch when one pass is shorter) until the time budget is spent, +
    acceptance over the sampled sequences' logit rows (repeated once per whole
    pass).  Scaled to draft tokens per second of the whole batch.  The inputs
    are regenerated from the seed of input set 0, so nothing the GPU wrote is
    used."""
    import oracle
    from threadpoolctl import threadpool_limits

    tree = w.name in wl.TREE_WORKLOADS
    long = w.name in wl.LONG_WORKLOADS
    case = wl.make_case(w, device=dev, seed_offset=0, with_logits=not (tree or long))
    np_ = lambda t: (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()
    if tree:
        case["parents"] = wl.make_tree(case["k_host"], device=dev, seed=w.ident)
        case.update(wl.make_tree_logits(w, case["k_host"], case["parents"], device=dev))
        parents = np_(case["parents"])
    sampled = w.name in wl.SAMPLED_WORKLOADS
    if sampled:
        dlog = np_(wl.make_draft_logits(case["logits"], case["k_host"], device=dev, seed=w.ident))
        ua, us = (np_(t) for t in wl.make_uniforms(case["T"], case["B"], device=dev, seed=w.ident))
    kp, vp = np_(case["k_pool"]), np_(case["v_pool"])
    bt, ctx, cu = np_(case["block_table"]), np_(case["ctx_lens"]), np_(case["cu_q"])
    qn = np_(case["q"])
    kn, vn = np_(case["k_new"]), np_(case["v_new"])
    logits = np_(case["logits"]) if "logits" in case else None
    drafts = np_(case["draft_ids"]) if "draft_ids" in case else None
    scale = 1.0 / math.sqrt(w.d)
    B, H = case["B"], w.Hkv
    pairs = [(b, g) for b in range(B) for g in range(H)]
    n_eval, t_attn = 0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if w.kv_dtype == "int8":
            # the INT8 cache holds oracle codes of the fp32 pool (cache fill, untimed)
            P = kp.shape[0]
            kc, ksc = oracle.kv_quant_int8(kp.reshape(-1, w.d))
            vc, vsc = oracle.kv_quant_int8(vp.reshape(-1, w.d))
            kp, vp = kc.reshape(kp.shape), vc.reshape(vp.shape)
            sc = dict(k_scale=ksc.reshape(P, H, 16), v_scale=vsc.reshape(P, H, 16))
            t0 = time.perf_counter()
            kp, vp, k_s, v_s = oracle.kv_append(kn, vn, kp, vp, bt, ctx, cu, "int8",
                                                sc["k_scale"], sc["v_scale"])
            sc = dict(k_scale=k_s, v_scale=v_s)
        else:
            sc = {}
            kp, vp, _, _ = oracle.kv_append(kn, vn, kp, vp, bt, ctx, cu, w.kv_dtype)
        t_append = time.perf_counter() - t0
        t0 = time.perf_counter()
        if tree:
            sc["draft_mask"] = oracle.ancestor_masks(parents, cu)
        while True:
            oracle.spec_verify_attn(qn, kp, vp, bt, ctx, cu, scale,
                                    select=[pairs[n_eval % len(pairs)]], **sc)
            n_eval += 1
            if time.perf_counter() - t0 > budget_s:
                break
        t_attn = time.perf_counter() - t0
        passes = n_eval / len(pairs)
        reps = max(1, int(passes))                  # acceptance passes
        seqs = sorted({b for b, _ in pairs[:min(n_eval, len(pairs))]})
        t0 = time.perf_counter()
        for b in ([] if long else seqs * reps):
            r0, r1 = int(cu[b]) + b, int(cu[b + 1]) + b + 1
            one = np.array([0, int(cu[b + 1] - cu[b])])
            if tree:
                _, n, _, path = oracle.accept_tree(logits[r0:r1], drafts[int(cu[b]):int(cu[b + 1])],
                                                   parents[int(cu[b]):int(cu[b + 1])], one)
                for pool in (kp, vp):
                    oracle.commit_path(pool, bt[b:b + 1], ctx[b:b + 1], one, n, path)
            elif sampled:
                q0, q1 = int(cu[b]), int(cu[b + 1])
                oracle.accept_stochastic(logits[r0:r1], dlog[q0:q1], drafts[q0:q1], one, 1.0,
                                         ua[q0:q1], us[b:b + 1])
            else:
                oracle.accept_prefix(logits[r0:r1], drafts[int(cu[b]):int(cu[b + 1])], one)
        t_acc = time.perf_counter() - t0
    frac_seqs = len(seqs) / B
    step_s = t_append + t_attn / passes + t_acc / (reps * frac_seqs)
    tokens = case["T"]
    return {
        "value": tokens / step_s, "unit": "verified draft tokens/s", "cores": 1, "kind": "oracle",
        "sample": (f"{n_eval} (sequence, kv-head) attention pairs, {passes:.2f} passes over the "
                   f"batch's {len(pairs)} ({t_attn:.1f} s), "
                   + ("" if long else f"acceptance{' and branch commit' if tree else ''} for "
                      f"{len(seqs)} of {B} sequences x {reps} ({t_acc:.1f} s), ")
                   + "the whole append once; scaled to one step of the full batch; numpy BLAS "
                     "limited to 1 thread"),
        "seconds_per_step_estimate": step_s,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mha7b")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0: enough to defeat the 256 MB MALL)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle attention")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    import token_verify_attention_amd as tva
    from token_verify_attention_amd import workloads as wl

    tva.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.WORKLOADS[args.workload]
    long = w.name in wl.LONG_WORKLOADS
    if w.vocab is None and not long:
        w = dataclasses.replace(w, vocab=128256, match_p=0.8)

    sets = [Inputs(tva, wl, w, 0, dev)]
    nsets = args.sets
    if not nsets:       # enough independent sets that the 256 MB MALL cannot hold them
        kvb0 = kv_bytes(w, sets[0].case["ctx_host"], sets[0].case["k_host"])
        nsets = max(1, min(4, math.ceil(3 * MALL_BYTES / max(kvb0, 1))))
    sets += [Inputs(tva, wl, w, s_, dev) for s_ in range(1, nsets)]
    nsets = len(sets)
    set_bytes = [kv_bytes(w, x.case["ctx_host"], x.case["k_host"]) for x in sets]
    set_tokens = [x.case["T"] for x in sets]
    kvb = sum(set_bytes) / nsets
    log(f"workload {w.name}: KV bytes per launch {kvb / 1e6:.1f} MB, {nsets} input set(s)")
    ctx, ks = sets[0].case["ctx_host"], sets[0].case["k_host"]
    max_pages = int(sets[0].case["block_table"].shape[1])
    T = sum(ks)

    stream = torch.cuda.current_stream(dev)
    for s in range(args.warmup):
        inp = sets[s % nsets]
        inp.append()
        inp.step_attn()
        inp.accept()
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    # Timed steps: nothing but the three calls per step on the stream (an event
    # between kernels costs a cache flush and a few microseconds of idle GPU).
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        inp = sets[s % nsets]
        inp.append()
        inp.step_attn()
        inp.accept()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    tokens_all = sum(set_tokens[s % nsets] for s in range(args.steps))
    value = tokens_all / (total_ms * 1e-3)
    T = tokens_all / args.steps

    # The attention kernel's average launch duration: the same number of
    # launches back to back on the same stream (same input-set rotation),
    # between one pair of HIP events.
    a_start, a_end = ev(), ev()
    torch.cuda.synchronize()
    a_start.record(stream)
    for s in range(args.steps):
        sets[s % nsets].attn()
    a_end.record(stream)
    torch.cuda.synchronize()
    attn_avg = a_start.elapsed_time(a_end) / args.steps
    # Per-launch distribution: each launch between its own pair of events
    # (the events add a little idle time between launches; the roofline
    # figures use the back-to-back average above).
    marks = [ev() for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for s in range(args.steps):
        sets[s % nsets].attn()
        marks[s + 1].record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]) * 1e3
    bytes_all = sum(set_bytes[s % nsets] for s in range(args.steps))
    kvb = bytes_all / args.steps
    achieved = kvb / (attn_avg * 1e-3) / 1e9
    traffic = measured_traffic(w.name, attn_avg)
    flops = sum(attn_flops(w, x.case["ctx_host"], x.case["k_host"]) for x in sets) / nsets
    tflops = flops / (attn_avg * 1e-3) / 1e12

    probe = copy_probe_gbps(dev)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype if w.kv_dtype != "int8" else "int8 KV, bf16 Q",
        "data": "synthetic (seeded torch Philox; no dataset)",
        "config": {
            "workload": (f"{w.name}: B={w.B}, Hq={w.Hq}, Hkv={w.Hkv}, d={w.d}, "
                         f"S={w.ctx}, k={w.k}"
                         f"{' drafts per step (step-level verification)' if long else ''}"
                         f"{' token-tree nodes' if w.name in wl.TREE_WORKLOADS else ''}, "
                         f"{w.kv_dtype} paged KV (16-token pages, random "
                         f"page permutation); "
                         f"{'no acceptance (a reward-model threshold)' if long else 'stochastic acceptance (rejection sampling, temperature 1) over fp32 target logits [sum(k_b+1), %d] and drafter logits [sum(k_b), %d]' % (w.vocab, w.vocab) if w.name in wl.SAMPLED_WORKLOADS else 'acceptance over fp32 logits [sum(k_b+1), %d]' % w.vocab}"),
            "global_batch": w.B, "seq_len": w.ctx if isinstance(w.ctx, int) else list(w.ctx),
            "drafts_per_seq": w.k if isinstance(w.k, int) else list(w.k),
            "parallelism": "single GPU", "input_sets_rotated": nsets,
        },
        "kv_bytes_per_launch": kvb,
        "kv_hbm_gbps": achieved,
        "kv_frac_of_peak": achieved / HBM_PEAK_GBPS,
        "attn_ms_avg": attn_avg,
        "attn_us_per_launch": {"p10": float(np.percentile(per_launch, 10)),
                               "p50": float(np.median(per_launch)),
                               "p90": float(np.percentile(per_launch, 90))},
        "attn_draft_tokens_per_s": T / (attn_avg * 1e-3),
        "draft_tokens_per_step": T,
        "other_bytes_per_launch": other_bytes(w, ctx, ks, max_pages),
        "copy_probe_gbps": probe,
        "attn_flops_per_launch": flops,
        "attn_tflops": tflops,
        "roofline": ({
            "bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": traffic and traffic["gbps"], "traffic_unit": "GB/s",
            "kernel": "verify_attn_rows_kernel",
            "traffic_bytes_per_launch": traffic and traffic["bytes"],
        } if long else {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic and traffic["gbps"],
            "kernel": "verify_attn_kernel",
            "traffic_bytes_per_launch": traffic and traffic["bytes"],
        }),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        del sets
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(wl, w, dev, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
