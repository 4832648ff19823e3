"""Seeded synthetic inputs for the verification hot path.

This module only draws random numbers and lays them out in the boundary's
formats; it performs none of the method's arithmetic (no attention, no
quantisation, no argmax).  Both the HIP path and the fp64 oracle consume what
it returns, so tests compare the two on identical bytes.

Random numbers come from torch's counter-based Philox generator on the device
the caller names, seeded per workload and per purpose, so a case is the same
on every run on the same device type.

Workloads (shapes of the pages' workloads; the serving datasets they stand in
for are not available, and none of their items are reproduced):

* ``tiny``        B=2, Hq=Hkv=4, d=64, S=128, k=4, fp32 Q/K/V ~ N(0,1);
                  acceptance logits [2*5, 1000], drafts agree with the target
                  argmax with probability 0.7 per position.
* ``mha7b``       B=8, Hq=Hkv=32, d=128, S=2048, k=4, bf16 ~ N(0,1).
* ``gqa8b``       B=32, Hq=32, Hkv=8, d=128, S=4096, k=8, bf16 ~ N(0,1), plus
                  k new K/V rows per sequence to append.
* ``gqa70b_int8`` B=16, Hq=64, Hkv=8, d=128, S=8192, k=4, K/V ~ N(0, 0.5) in
                  fp32 (quantised to INT8 by the code under test), Q bf16.
* ``gqa70b_int8_tp8`` one GPU's share of ``gqa70b_int8`` under 8-way tensor
                  parallelism over kv heads: B=16, Hq=8, Hkv=1, otherwise the
                  same (16 (sequence, kv head) pairs, each split over many
                  workgroups).
* ``ragged``      B=64, S_b ~ U[256, 16384], k_b ~ U{1..8}, Hq=32, Hkv=8,
                  d=128, bf16; acceptance logits [sum(k_b+1), 128256] ~ N(0,1),
                  drafts agree with the target argmax with probability 0.8.
* ``tree8b``      the 8B GQA shape with a token tree of 8 nodes per sequence
                  instead of a chain (B=32, Hq=32, Hkv=8, d=128, S=4096, bf16);
                  acceptance logits [sum(k_b+1), 128256], node tokens agree
                  with the target argmax at their parent with probability 0.8.

* ``prm7b_step``  step-level verification of long speculated steps: the
                  attention shape of a 7B process reward model (Qwen2.5-Math-
                  7B: Hq=28, Hkv=4, d=128) scoring a 128-token step per
                  sequence, B=16, S=4096, bf16 ~ N(0,1).
* ``prm7b_step_b1`` the same for one sequence (B=1): the latency of scoring
                  a single reasoning step, where the row blocks alone would
                  occupy 16 CUs.
* ``ragged_sampled`` the ragged serving batch with stochastic acceptance:
                  drafter logits [T, 128256] = the target row's logits plus
                  N(0, 0.5^2) noise, temperature 1, uniforms u_accept [T] and
                  u_sample [B] from U[0, 1).

Token trees (``make_tree``): node i's parent is node i-1 with probability 1/2,
else uniform over {-1, 0, .., i-2} (-1: a child of the last committed token),
so trees mix deep chains and side branches the way dynamic drafters build
them.  ``make_tree_logits`` plants each row's maximum as for chains and gives
node i the planted token of its parent's row (row 0 for the root) with the
workload's agreement probability, else a different token.

Every workload uses 16-token pages laid out as [P, Hkv, 16, d] with a random
page permutation; unused block-table entries are -1.  The pool holds exactly
sum_b ceil((S_b + k_b) / 16) pages.  Slots past S_b + k_b in a sequence's last
page hold ordinary draws, or NaN when ``poison=True``.

Logit rows are drawn with the argmax planted at a chosen index without
computing any maximum: the top value is drawn from the law of the maximum of V
i.i.d. N(0,1) variables (inverse CDF of U**(1/V)) and the other V-1 values from
N(0,1) truncated below it (inverse CDF of U * Phi(top)).  That is exactly the
law of V i.i.d. normals conditioned on where their maximum sits.
"""
from dataclasses import dataclass
from typing import Optional, Tuple, Union

import torch

PAGE = 16


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    ctx: Union[int, Tuple[int, int]]          # S, or inclusive uniform range
    k: Union[int, Tuple[int, int]]            # k, or inclusive uniform range
    kv_dtype: str                             # 'f32' | 'bf16' | 'int8'
    q_dtype: str                              # 'f32' | 'bf16'
    sigma: float = 1.0
    vocab: Optional[int] = None
    match_p: Optional[float] = None
    append: bool = False
    ident: int = 0                            # seed namespace


WORKLOADS = {
    "tiny": Workload("tiny", 2, 4, 4, 64, 128, 4, "f32", "f32", 1.0, 1000, 0.7, False, 1),
    "mha7b": Workload("mha7b", 8, 32, 32, 128, 2048, 4, "bf16", "bf16", ident=2),
    "gqa8b": Workload("gqa8b", 32, 32, 8, 128, 4096, 8, "bf16", "bf16", append=True, ident=3),
    "gqa70b_int8": Workload("gqa70b_int8", 16, 64, 8, 128, 8192, 4, "int8", "bf16", 0.5, ident=4),
    "gqa70b_int8_tp8": Workload("gqa70b_int8_tp8", 16, 8, 1, 128, 8192, 4, "int8", "bf16", 0.5,
                                ident=9),
    "ragged": Workload("ragged", 64, 32, 8, 128, (256, 16384), (1, 8), "bf16", "bf16",
                       1.0, 128256, 0.8, ident=5),
    "tree8b": Workload("tree8b", 32, 32, 8, 128, 4096, 8, "bf16", "bf16", 1.0, 128256, 0.8,
                       append=True, ident=6),
    "ragged_sampled": Workload("ragged_sampled", 64, 32, 8, 128, (256, 16384), (1, 8), "bf16",
                               "bf16", 1.0, 128256, 0.8, ident=7),
    "prm7b_step": Workload("prm7b_step", 16, 28, 4, 128, 4096, 128, "bf16", "bf16", append=True,
                           ident=8),
    "prm7b_step_b1": Workload("prm7b_step_b1", 1, 28, 4, 128, 4096, 128, "bf16", "bf16",
                              append=True, ident=10),
}

SAMPLED_WORKLOADS = ("ragged_sampled",)
LONG_WORKLOADS = ("prm7b_step", "prm7b_step_b1")

TREE_WORKLOADS = ("tree8b",)

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randint(lo, hi, n, g, device):
    return torch.randint(lo, hi + 1, (n,), generator=g, device=device, dtype=torch.int64)


def _normal(shape, sigma, dtype, g, device):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)                       # exact for sigma a power of two
    return x if dtype == torch.float32 else x.to(dtype)


def make_lengths(w: Workload, seed_offset=0, device="cpu"):
    """ctx_lens [B] and k [B] as int64 tensors on ``device``."""
    g = _gen(device, 1000 + w.ident + 97 * seed_offset)
    if isinstance(w.ctx, tuple):
        ctx = _randint(w.ctx[0], w.ctx[1], w.B, g, device)
    else:
        ctx = torch.full((w.B,), w.ctx, dtype=torch.int64, device=device)
    if isinstance(w.k, tuple):
        k = _randint(w.k[0], w.k[1], w.B, g, device)
    else:
        k = torch.full((w.B,), w.k, dtype=torch.int64, device=device)
    return ctx, k


def make_case(w: Workload, device="cpu", seed_offset=0, poison=False, ctx=None, k=None,
              with_logits=True, extra_pages=0):
    """Build one synthetic batch.  Returns a dict of tensors on ``device``.

    Keys: ctx_lens int32 [B], cu_q int32 [B+1], q [T, Hq, d], k_pool/v_pool
    [P, Hkv, 16, d] (fp32 source values for INT8 workloads), block_table
    int32 [B, max_pages] (-1 padded), k_new/v_new [T, Hkv, d], and, when the
    workload has a vocabulary, logits f32 [T+B, V], draft_ids int32 [T] and
    planted int64 [T+B] (the index each logit row's maximum was planted at).
    ``ctx``/``k`` override the drawn lengths (lists of ints).
    ``extra_pages`` adds unreferenced pages to the pool.
    """
    if ctx is None:
        ctx, k = make_lengths(w, seed_offset, device)
    else:
        ctx = torch.as_tensor(ctx, dtype=torch.int64, device=device)
        k = torch.as_tensor(k, dtype=torch.int64, device=device)
    B = ctx.numel()
    ctx_h = [int(v) for v in ctx.cpu()]
    k_h = [int(v) for v in k.cpu()]
    npages = [-(-(c + kk) // PAGE) for c, kk in zip(ctx_h, k_h)]
    P = sum(npages) + extra_pages
    max_pages = max(npages + [1])
    T = sum(k_h)

    gi = _gen(device, 1000 + w.ident + 97 * seed_offset + 7)
    gp = _gen(device, 2000 + w.ident + 97 * seed_offset)
    src_dt = torch.float32 if w.kv_dtype in ("f32", "int8") else TORCH_DTYPE[w.kv_dtype]

    perm = torch.randperm(P, generator=gp, device=device).to(torch.int32)
    block_table = torch.full((B, max_pages), -1, dtype=torch.int32, device=device)
    off = 0
    for b in range(B):
        block_table[b, : npages[b]] = perm[off: off + npages[b]]
        off += npages[b]

    k_pool = _normal((P, w.Hkv, PAGE, w.d), w.sigma, src_dt, gi, device)
    v_pool = _normal((P, w.Hkv, PAGE, w.d), w.sigma, src_dt, gi, device)
    q = _normal((T, w.Hq, w.d), w.sigma, TORCH_DTYPE[w.q_dtype], gi, device)
    k_new = _normal((T, w.Hkv, w.d), w.sigma, src_dt, gi, device)
    v_new = _normal((T, w.Hkv, w.d), w.sigma, src_dt, gi, device)

    if poison:
        for b in range(B):
            used = ctx_h[b] + k_h[b]
            last = npages[b] - 1
            if used % PAGE:
                pg = int(block_table[b, last])
                k_pool[pg, :, used % PAGE:, :] = float("nan")
                v_pool[pg, :, used % PAGE:, :] = float("nan")
        if extra_pages:
            unused = perm[off:].long()
            k_pool[unused] = float("nan")
            v_pool[unused] = float("nan")

    cu_q = torch.zeros(B + 1, dtype=torch.int32, device=device)
    cu_q[1:] = torch.cumsum(k, 0).to(torch.int32)
    case = dict(
        workload=w, ctx_lens=ctx.to(torch.int32), cu_q=cu_q, q=q, k_pool=k_pool, v_pool=v_pool,
        block_table=block_table, k_new=k_new, v_new=v_new, T=T, B=B, max_len=max(
            c + kk for c, kk in zip(ctx_h, k_h)) if B else 0, max_q=max(k_h) if B else 0,
        ctx_host=ctx_h, k_host=k_h,
    )
    if with_logits and w.vocab is not None:
        case.update(make_logits(w, k_h, device, seed_offset))
    return case


def planted_rows(n_rows, V, planted, g, device, chunk=64):
    """[n_rows, V] float32 rows of i.i.d. N(0,1) whose maximum sits at
    ``planted[r]``, drawn without computing any maximum (see module doc)."""
    out = torch.empty((n_rows, V), dtype=torch.float32, device=device)
    for r0 in range(0, n_rows, chunk):
        r1 = min(n_rows, r0 + chunk)
        n = r1 - r0
        u_top = torch.rand((n, 1), generator=g, device=device, dtype=torch.float64)
        # U**(1/V) = 1 - a with a = -expm1(log(U)/V); Phi^-1(1 - a) = -Phi^-1(a)
        a = -torch.expm1(torch.log(u_top) / V)
        top = -torch.special.ndtri(a)
        u = torch.rand((n, V), generator=g, device=device, dtype=torch.float64)
        rest = torch.special.ndtri(u * torch.special.ndtr(top))
        rest.scatter_(1, planted[r0:r1].view(-1, 1), top)
        out[r0:r1] = rest.to(torch.float32)
    return out


def make_logits(w: Workload, k_h, device="cpu", seed_offset=0):
    """Acceptance inputs: logits [sum(k_b+1), V], planted target ids, drafts."""
    g = _gen(device, 3000 + w.ident + 97 * seed_offset)
    B = len(k_h)
    rows = sum(k_h) + B
    V = w.vocab
    planted = torch.randint(0, V, (rows,), generator=g, device=device, dtype=torch.int64)
    logits = planted_rows(rows, V, planted, g, device)
    T = sum(k_h)
    seq_of = torch.repeat_interleave(torch.arange(B, device=device),
                                     torch.as_tensor(k_h, dtype=torch.int64, device=device))
    draft = planted[torch.arange(T, device=device) + seq_of]
    if T:
        miss = torch.rand(T, generator=g, device=device) >= w.match_p
        shift = 1 + torch.randint(0, V - 1, (T,), generator=g, device=device, dtype=torch.int64)
        draft = torch.where(miss, (draft + shift) % V, draft)
    return dict(logits=logits, draft_ids=draft.to(torch.int32), planted=planted)


def make_tree(k_h, device="cpu", seed=0, p_chain=0.5):
    """Parent arrays of one token tree per sequence, concatenated: int32 [T]."""
    g = _gen("cpu", 4000 + seed)
    out = []
    for k in k_h:
        for i in range(k):
            u = float(torch.rand((), generator=g))
            if i > 0 and u < p_chain:
                out.append(i - 1)
            else:
                out.append(int(torch.randint(-1, max(i - 1, 0), (), generator=g)) if i > 1 else -1)
    return torch.tensor(out, dtype=torch.int32, device=device)


def make_tree_logits(w: Workload, k_h, parents, device="cpu", seed_offset=0):
    """Tree acceptance inputs: logits [sum(k_b+1), V] with planted row maxima
    and node tokens that copy the planted token of their parent's row with
    probability ``w.match_p`` (else a different token)."""
    g = _gen(device, 5000 + w.ident + 97 * seed_offset)
    B = len(k_h)
    rows = sum(k_h) + B
    V = w.vocab
    planted = torch.randint(0, V, (rows,), generator=g, device=device, dtype=torch.int64)
    logits = planted_rows(rows, V, planted, g, device)
    T = sum(k_h)
    seq_of = torch.repeat_interleave(torch.arange(B, device=device),
                                     torch.as_tensor(k_h, dtype=torch.int64, device=device))
    starts = torch.zeros(B, dtype=torch.int64, device=device)
    if B:
        starts[1:] = torch.cumsum(torch.as_tensor(k_h, dtype=torch.int64, device=device), 0)[:-1]
    par = parents.to(device=device, dtype=torch.int64)
    # row of the parent: sequence row base (start + b) + 1 + parent
    parent_row = starts[seq_of] + seq_of + 1 + par if T else par
    draft = planted[parent_row] if T else planted[:0]
    if T:
        miss = torch.rand(T, generator=g, device=device) >= w.match_p
        shift = 1 + torch.randint(0, V - 1, (T,), generator=g, device=device, dtype=torch.int64)
        draft = torch.where(miss, (draft + shift) % V, draft)
    return dict(logits=logits, draft_ids=draft.to(torch.int32), planted=planted)


def make_draft_logits(logits, k_h, device="cpu", seed=0, noise=0.5):
    """Drafter logits [T, V]: row j of sequence b is the target's row j
    (cu_q[b] + b + j) plus N(0, noise^2) noise."""
    g = _gen(device, 6000 + seed)
    B = len(k_h)
    rows = []
    base = 0
    for b, k in enumerate(k_h):
        rows.append(torch.arange(base + b, base + b + k, device=device))
        base += k
    idx = torch.cat(rows) if rows else torch.zeros(0, dtype=torch.int64, device=device)
    out = logits[idx].clone()
    out.add_(torch.randn(out.shape, generator=g, device=device, dtype=torch.float32), alpha=noise)
    return out


def make_uniforms(T, B, device="cpu", seed=0):
    """u_accept [T] and u_sample [B] from U[0, 1) (float32)."""
    g = _gen(device, 7000 + seed)
    return (torch.rand(T, generator=g, device=device, dtype=torch.float32),
            torch.rand(B, generator=g, device=device, dtype=torch.float32))
