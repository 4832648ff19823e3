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
  model's threshold is not part of this path); --workload prm7b_step_b1 is the
  same for one sequence (the latency of scoring one step).

Default workload: the ragged serving batch -- B=64, S_b ~ U[256, 16384],
k_b ~ U{1..8}, Hq=32, Hkv=8, d=128, bf16 paged KV (16-token pages, random page
permutation), acceptance over fp32 logits [sum(k_b+1), 128256] with drafts
agreeing with the target argmax with probability 0.8 -- the largest of the
single-GPU workloads.  The same run also times the other workloads (tiny,
7B MHA, 8B GQA, 70B-shaped INT8) under "configs", and a streaming-read probe
kernel as the achievable ceiling of the KV stream.

Prints ONE JSON line.  `value` is verified draft tokens per second for whole
steps (inputs resident in HBM); `goodput_accepted_tokens_per_s` counts the
tokens the steps emit (sum of n_b + 1); `roofline` is the attention kernel's
KV bytes over its own average launch time against 8 TB/s; `cpu_baseline` is
the fp64 oracle on the host's cores.  The attention kernel's average launch
time comes from the same number of back-to-back launches of the attention
call alone (sva_spec_verify_attn, no append) after the timed steps, between
one pair of HIP events on its stream; `roofline.traffic` is HBM traffic from
committed rocprofv3 counter readings (null when they no longer match the
kernel's sources).

The CPU baseline's worker processes are forked, with the host copy of the
workload, before anything touches the GPU; they never use it.
"""
import argparse
import dataclasses
import json
import math
import multiprocessing
import os
import sys
import time

import numpy as np
import torch

METRIC = "verify-attn KV HBM GB/s (% of peak) and verified draft tokens/sec, 1 GPU"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
MFMA_BF16_PEAK_TFLOPS = 2500.0
MAX_CPU_WORKERS = 16
EXTRA_CONFIGS = ("tiny", "mha7b", "gqa8b", "gqa70b_int8", "prm7b_step", "prm7b_step_b1")
CONFIG_MIN_STEPS = 50


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


def step_workload(wl, name):
    """The workload as the step runs it: shapes without a vocabulary get the
    ragged batch's (128256 tokens, 80 % agreement) for their acceptance."""
    w = wl.WORKLOADS[name]
    if w.vocab is None and name not in wl.LONG_WORKLOADS:
        w = dataclasses.replace(w, vocab=128256, match_p=0.8)
    return w


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host's cores
# ---------------------------------------------------------------------------

_HOST = {}          # the host copy of the workload; inherited by forked workers


def _attn_share(share, budget_s):
    """Worker: the oracle's attention over this worker's (sequence, kv-head)
    pairs, taken in order and repeated until the time budget is spent."""
    import oracle
    from threadpoolctl import threadpool_limits
    h = _HOST
    n = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            oracle.spec_verify_attn(h["q"], h["k"], h["v"], h["bt"], h["ctx"], h["cu"],
                                    h["scale"], select=[share[n % len(share)]], **h["kw"])
            n += 1
            if time.perf_counter() - t0 > budget_s:
                break
    return n, time.perf_counter() - t0


class CpuBaseline:
    """The oracle as it stands, on the same workload drawn on the host (same
    recipe and seeds, the host's generator), timed per step:
      append     oracle.kv_append of the whole batch, once, one core;
      attention  every (sequence, kv-head) pair, split over `cores` forked
                 worker processes (pair i to worker i mod cores), each
                 repeating its share until its time budget is spent; a pass
                 takes as long as the slowest worker's share;
      acceptance every sequence (greedy prefix, tree walk + branch commit, or
                 rejection sampling), one core, repeated until 0.5 s is spent.
    Built before the GPU is touched (the workers are forked here)."""

    def __init__(self, wl, w, cores):
        import oracle
        from threadpoolctl import threadpool_limits
        self.w, self.cores = w, cores
        tree = w.name in wl.TREE_WORKLOADS
        long = w.name in wl.LONG_WORKLOADS
        sampled = w.name in wl.SAMPLED_WORKLOADS
        self.long = long
        t0 = time.perf_counter()
        case = wl.make_case(w, device="cpu", seed_offset=0, with_logits=not (tree or long))
        np_ = lambda t: (t.float() if t.dtype == torch.bfloat16 else t).numpy()
        if tree:
            case["parents"] = wl.make_tree(case["k_host"], device="cpu", seed=w.ident)
            case.update(wl.make_tree_logits(w, case["k_host"], case["parents"], device="cpu"))
        bt, ctx, cu = np_(case["block_table"]), np_(case["ctx_lens"]), np_(case["cu_q"])
        kp, vp = np_(case.pop("k_pool")), np_(case.pop("v_pool"))
        kn, vn = np_(case["k_new"]), np_(case["v_new"])
        self.T, self.B = case["T"], case["B"]
        self.gen_s = time.perf_counter() - t0
        with threadpool_limits(limits=1):
            kw = {}
            if w.kv_dtype == "int8":
                # the INT8 cache holds oracle codes of the fp32 pool (cache fill, untimed)
                P, H = kp.shape[:2]
                kc, ksc = oracle.kv_quant_int8(kp.reshape(-1, w.d))
                vc, vsc = oracle.kv_quant_int8(vp.reshape(-1, w.d))
                t0 = time.perf_counter()
                kp, vp, ksc, vsc = oracle.kv_append(kn, vn, kc.reshape(kp.shape),
                                                    vc.reshape(vp.shape), bt, ctx, cu, "int8",
                                                    ksc.reshape(P, H, 16), vsc.reshape(P, H, 16))
                kw = dict(k_scale=ksc, v_scale=vsc)
            else:
                t0 = time.perf_counter()
                kp, vp, _, _ = oracle.kv_append(kn, vn, kp, vp, bt, ctx, cu, w.kv_dtype)
            self.t_append = time.perf_counter() - t0
            if tree:
                kw["draft_mask"] = oracle.ancestor_masks(np_(case["parents"]), cu)
        self._acc_args = (wl, case, np_, kp, vp, bt, ctx, cu, tree, long, sampled)
        _HOST.update(q=np_(case["q"]), k=kp, v=vp, bt=bt, ctx=ctx, cu=cu,
                     scale=1.0 / math.sqrt(w.d), kw=kw)
        self.pairs = [(b, g) for b in range(self.B) for g in range(w.Hkv)]
        self.pool = multiprocessing.get_context("fork").Pool(cores)

    def _time_acceptance(self, wl, case, np_, kp, vp, bt, ctx, cu, tree, long, sampled):
        import oracle
        if long:
            return 0.0, 0
        w = self.w
        logits, drafts = np_(case["logits"]), np_(case["draft_ids"])
        if sampled:
            dlog = np_(wl.make_draft_logits(case["logits"], case["k_host"], device="cpu",
                                            seed=w.ident))
            ua, us = (np_(t) for t in wl.make_uniforms(self.T, self.B, device="cpu",
                                                       seed=w.ident))
        parents = np_(case["parents"]) if tree else None
        reps, t0 = 0, time.perf_counter()
        while True:
            for b in range(self.B):
                r0, r1 = int(cu[b]) + b, int(cu[b + 1]) + b + 1
                q0, q1 = int(cu[b]), int(cu[b + 1])
                one = np.array([0, q1 - q0])
                if tree:
                    _, n, _, path = oracle.accept_tree(logits[r0:r1], drafts[q0:q1],
                                                       parents[q0:q1], one)
                    for pool in (kp, vp):       # after the attention: the pools may change
                        oracle.commit_path(pool, bt[b:b + 1], ctx[b:b + 1], one, n, path)
                elif sampled:
                    oracle.accept_stochastic(logits[r0:r1], dlog[q0:q1], drafts[q0:q1], one, 1.0,
                                             ua[q0:q1], us[b:b + 1])
                else:
                    oracle.accept_prefix(logits[r0:r1], drafts[q0:q1], one)
            reps += 1
            if time.perf_counter() - t0 > 0.5:
                break
        return (time.perf_counter() - t0) / reps, reps

    def run(self, budget_s):
        shares = [self.pairs[i::self.cores] for i in range(self.cores)]
        shares = [s for s in shares if s]
        res = self.pool.starmap(_attn_share, [(s, budget_s) for s in shares])
        self.pool.close()
        self.pool.join()
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            self.t_accept, self.accept_reps = self._time_acceptance(*self._acc_args)
        # seconds per pass over each worker's share; the pass ends with the slowest
        per_pass = [t / (n / len(s)) for (n, t), s in zip(res, shares)]
        t_attn = max(per_pass)
        n_eval = sum(n for n, _ in res)
        step_s = self.t_append + t_attn + self.t_accept
        w = self.w
        return {
            "value": self.T / step_s, "unit": "verified draft tokens/s", "cores": len(shares),
            "kind": "oracle",
            "sample": (f"{n_eval} (sequence, kv-head) attention pairs over {len(shares)} worker "
                       f"processes (each repeating its share of the batch's {len(self.pairs)} "
                       f"pairs for {budget_s:.0f} s; a pass takes {t_attn * 1e3:.1f} ms, the slowest "
                       f"share), the whole append once ({self.t_append * 1e3:.1f} ms, one core)"
                       + ("" if self.long else
                          f", acceptance of all {self.B} sequences x {self.accept_reps} "
                          f"({self.t_accept * 1e3:.2f} ms each, one core)")
                       + f"; inputs drawn on the host with the workload's recipe and seeds; "
                         f"numpy BLAS limited to 1 thread per process"),
            "seconds_per_step_estimate": step_s,
        }


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------

class Inputs:
    """One resident input set and the prepared calls of one step."""

    def __init__(self, tva, wl, w, seed_offset, dev, path=0):
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
        self.has_accept = not long
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
            self.attn = tva.prepare_spec_verify_attn(self.batch, case["q"], self.kv, self.out,
                                                     path=path)
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
                    self.batch, case["q"], self.kv, case["k_new"], case["v_new"], self.out,
                    path=path)
                self.append = lambda stream=None: None

    def step(self):
        self.append()
        self.step_attn()
        self.accept()

    def emitted_tokens(self):
        """Tokens the step emits: sum over sequences of n_b + 1 (the accepted
        drafts and the target's token after them).  The step's inputs are the
        same every time, so every step of this set emits the same count."""
        return int(self.alen.sum().item()) + self.case["B"] if self.has_accept else 0


def measure(tva, wl, w, dev, steps, warmup, sets=0, path=0):
    """Time `steps` whole steps (inputs resident in HBM), then the same number
    of back-to-back attention launches and the same launches one by one."""
    inp0 = Inputs(tva, wl, w, 0, dev, path)
    nsets = sets
    if not nsets:       # enough independent sets that the 256 MB MALL cannot hold them
        kvb0 = kv_bytes(w, inp0.case["ctx_host"], inp0.case["k_host"])
        nsets = max(1, min(4, math.ceil(3 * MALL_BYTES / max(kvb0, 1))))
    ins = [inp0] + [Inputs(tva, wl, w, s_, dev, path) for s_ in range(1, nsets)]
    set_bytes = [kv_bytes(w, x.case["ctx_host"], x.case["k_host"]) for x in ins]
    set_tokens = [x.case["T"] for x in ins]
    stream = torch.cuda.current_stream(dev)
    for s in range(warmup):
        ins[s % nsets].step()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # Timed steps: nothing but the calls of each step on the stream (an event
    # between kernels costs a cache flush and a few microseconds of idle GPU).
    t0, t1 = ev(), ev()
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(steps):
        ins[s % nsets].step()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    emitted = [x.emitted_tokens() for x in ins]
    tokens_all = sum(set_tokens[s % nsets] for s in range(steps))
    emitted_all = sum(emitted[s % nsets] for s in range(steps))
    # attention alone, back to back, same rotation
    a0, a1 = ev(), ev()
    torch.cuda.synchronize()
    a0.record(stream)
    for s in range(steps):
        ins[s % nsets].attn()
    a1.record(stream)
    torch.cuda.synchronize()
    attn_ms = a0.elapsed_time(a1) / steps
    marks = [ev() for _ in range(steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for s in range(steps):
        ins[s % nsets].attn()
        marks[s + 1].record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]) * 1e3
    kvb = sum(set_bytes[s % nsets] for s in range(steps)) / steps
    flops = sum(attn_flops(w, x.case["ctx_host"], x.case["k_host"]) for x in ins) / nsets
    ctx, ks = ins[0].case["ctx_host"], ins[0].case["k_host"]
    r = {
        "nsets": nsets, "ms_per_step": total_ms / steps,
        "tokens_per_s": tokens_all / (total_ms * 1e-3),
        "draft_tokens_per_step": tokens_all / steps,
        "emitted_tokens_per_step": emitted_all / steps,
        "goodput": emitted_all / (total_ms * 1e-3),
        "attn_ms": attn_ms,
        "attn_us_per_launch": {"p10": float(np.percentile(per_launch, 10)),
                               "p50": float(np.median(per_launch)),
                               "p90": float(np.percentile(per_launch, 90))},
        "kv_bytes": kvb, "kv_gbps": kvb / (attn_ms * 1e-3) / 1e9,
        "flops": flops, "tflops": flops / (attn_ms * 1e-3) / 1e12,
        "other_bytes": other_bytes(w, ctx, ks, int(ins[0].case["block_table"].shape[1])),
    }
    del ins, inp0
    torch.cuda.empty_cache()
    return r


def probe_ceiling(tva, dev, num_cus, nbytes=1 << 30, reps=10, trials=3):
    """Best read rate of the streaming-read probe kernel over a few launch
    shapes (a 1 GiB buffer, 4x the MALL; each shape the best of `trials` runs
    of `reps` launches, one run varying by a few percent), the same over 4 KB
    pages in a scattered order (the KV cache's access pattern), and a plain
    torch device copy."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(65536 * 4, dtype=torch.int32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    shapes = ([(0, num_cus * k) for k in (4, 8, 16)] + [(1, num_cus), (1, 2 * num_cus)]
              + [(2, num_cus), (2, 2 * num_cus)])
    rates = {}
    for mode, nwg in shapes:
        tva.stream_read_probe(buf, mode, nwg, sink)
        torch.cuda.synchronize()
        best_rate = 0.0
        for _ in range(trials):
            e0, e1 = ev(), ev()
            e0.record()
            for _ in range(reps):
                tva.stream_read_probe(buf, mode, nwg, sink)
            e1.record()
            torch.cuda.synchronize()
            best_rate = max(best_rate, nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        rates[f"{('regs', 'lds', 'lds_pages')[mode]}_wg{nwg}"] = best_rate
    b = torch.empty_like(buf)
    b.copy_(buf)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(reps):
        b.copy_(buf)
    e1.record()
    torch.cuda.synchronize()
    copy = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, b
    torch.cuda.empty_cache()
    contiguous = {k: v for k, v in rates.items() if "pages" not in k}
    pages = {k: v for k, v in rates.items() if "pages" in k}
    best = max(contiguous, key=contiguous.get)
    best_pages = max(pages, key=pages.get)
    return {"read_gbps": rates[best], "best_shape": best,
            "page_read_gbps": rates[best_pages], "best_page_shape": best_pages, "shapes": rates,
            "torch_copy_gbps_read_plus_write": copy}


def describe(w, wl):
    long = w.name in wl.LONG_WORKLOADS
    if long:
        acc = "no acceptance (a reward-model threshold)"
    elif w.name in wl.SAMPLED_WORKLOADS:
        acc = ("stochastic acceptance (rejection sampling, temperature 1) over fp32 target logits "
               f"[sum(k_b+1), {w.vocab}] and drafter logits [sum(k_b), {w.vocab}]")
    else:
        acc = f"acceptance over fp32 logits [sum(k_b+1), {w.vocab}]"
    return (f"{w.name}: B={w.B}, Hq={w.Hq}, Hkv={w.Hkv}, d={w.d}, S={w.ctx}, k={w.k}"
            f"{' drafts per step (step-level verification)' if long else ''}"
            f"{' token-tree nodes' if w.name in wl.TREE_WORKLOADS else ''}, "
            f"{w.kv_dtype} paged KV (16-token pages, random page permutation); {acc}")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ragged")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0: enough to defeat the 256 MB MALL)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle attention per CPU worker")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other workloads (the 'configs' key)")
    ap.add_argument("--path", type=int, default=0,
                    help="attention inner path: 0 default (MFMA for bf16 / INT8), 1 VALU")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    from token_verify_attention_amd import workloads as wl
    w = step_workload(wl, args.workload)
    long = w.name in wl.LONG_WORKLOADS

    # The CPU baseline's host inputs and worker processes come first: the
    # workers are forked before this process touches the GPU.
    cpu = None
    if not args.no_cpu_baseline:
        cores = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
        log(f"cpu baseline: host inputs and {cores} workers ...")
        cpu = CpuBaseline(wl, w, cores)

    import token_verify_attention_amd as tva
    tva.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count

    log(f"workload {w.name}: timing {args.steps} steps")
    m = measure(tva, wl, w, dev, args.steps, args.warmup, args.sets, args.path)
    traffic = measured_traffic(w.name, m["attn_ms"])
    probe = probe_ceiling(tva, dev, num_cus)
    log(f"probe ceiling {probe['read_gbps']:.0f} GB/s ({probe['best_shape']}); "
        f"scattered 4 KB pages {probe['page_read_gbps']:.0f} GB/s")

    configs = {}
    if not args.no_configs and w.name == "ragged":
        for name in EXTRA_CONFIGS:
            log(f"config {name}")
            wc = step_workload(wl, name)
            # at least 50 steps: the configs' launches are short and 20 of them vary
            r = measure(tva, wl, wc, dev, max(args.steps, CONFIG_MIN_STEPS), max(args.warmup, 5))
            configs[name] = {
                "workload": describe(wc, wl),
                "attn_us": r["attn_ms"] * 1e3, "kv_bytes_per_launch": r["kv_bytes"],
                "kv_hbm_gbps": r["kv_gbps"], "kv_frac_of_peak": r["kv_gbps"] / HBM_PEAK_GBPS,
                "kv_frac_of_probe": r["kv_gbps"] / probe["read_gbps"],
                "kv_frac_of_page_probe": r["kv_gbps"] / probe["page_read_gbps"],
                "attn_us_per_launch": r["attn_us_per_launch"],
                "ms_per_step": r["ms_per_step"],
                "verified_draft_tokens_per_s": r["tokens_per_s"],
                "goodput_accepted_tokens_per_s": r["goodput"],
                "emitted_tokens_per_step": r["emitted_tokens_per_step"],
                "input_sets_rotated": r["nsets"],
            }
            if name == "tiny":
                configs[name]["note"] = ("0.56 MB working set: launch-bound, far below the time "
                                         "70 % of 8 TB/s would take (0.1 us)")
            if name in wl.LONG_WORKLOADS:       # MFMA-bound; no acceptance in the step
                configs[name].update({
                    "attn_flops_per_launch": r["flops"], "attn_tflops": r["tflops"],
                    "mfma_frac_of_peak": r["tflops"] / MFMA_BF16_PEAK_TFLOPS,
                    "goodput_accepted_tokens_per_s": None, "emitted_tokens_per_step": None})

    achieved = m["kv_gbps"]
    result = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype if w.kv_dtype != "int8" else "int8 KV, bf16 Q",
        "data": "synthetic (seeded torch Philox; no dataset)",
        "config": {
            "workload": describe(w, wl),
            "global_batch": w.B, "seq_len": w.ctx if isinstance(w.ctx, int) else list(w.ctx),
            "drafts_per_seq": w.k if isinstance(w.k, int) else list(w.k),
            "parallelism": "single GPU", "input_sets_rotated": m["nsets"],
            "attention_path": {0: "default", 1: "VALU", 2: "MFMA"}[args.path],
        },
        "goodput_accepted_tokens_per_s": m["goodput"],
        "emitted_tokens_per_step": m["emitted_tokens_per_step"],
        "draft_tokens_per_step": m["draft_tokens_per_step"],
        "kv_bytes_per_launch": m["kv_bytes"],
        "kv_hbm_gbps": achieved,
        "kv_frac_of_peak": achieved / HBM_PEAK_GBPS,
        "kv_frac_of_probe": achieved / probe["read_gbps"],
        "kv_frac_of_page_probe": achieved / probe["page_read_gbps"],
        "attn_ms_avg": m["attn_ms"],
        "attn_us_per_launch": m["attn_us_per_launch"],
        "attn_draft_tokens_per_s": m["draft_tokens_per_step"] / (m["attn_ms"] * 1e-3),
        "other_bytes_per_launch": m["other_bytes"],
        "probe": probe,
        "attn_flops_per_launch": m["flops"],
        "attn_tflops": m["tflops"],
        "roofline": ({
            "bound": "mfma", "achieved": m["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": m["tflops"] / MFMA_BF16_PEAK_TFLOPS,
            "traffic": traffic and traffic["gbps"], "traffic_unit": "GB/s",
            "kernel": "verify_attn_rows_kernel",
            "traffic_bytes_per_launch": traffic and traffic["bytes"],
        } if long else {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic and traffic["gbps"],
            "kernel": "verify_attn_kernel",
            "traffic_bytes_per_launch": traffic and traffic["bytes"],
        }),
        "configs": configs,
        "cpu_baseline": None,
    }
    if cpu is not None:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu.run(args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
