"""Plain, slow, fp64 CPU oracle for the speculative-verification hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path: the two
share no code, no tables and no pre- or post-processing.

What each function follows (pages cited by title and section):

* ``spec_verify_attn`` -- causal multi-query attention of the k draft queries of
  each sequence over its paged KV cache.  "Decoding Speculative Decoding from
  First Principles", sections "Speculating to get sequence parallelism during
  decode" (the target scores every draft in one prefill-style pass) and the
  prerequisites section (causal masked attention); "CXL-SpecKV", key
  observation (1) (token t reads positions 0..t-1) and the memory-hierarchy
  section (4 KB pages).  Written as the plain softmax-attention definition,
  because split-KV with an online softmax reaches exactly that result.
* ``kv_quant_int8`` / ``dequant_int8`` -- "CXL-SpecKV", Algorithm 2 (KV-Cache
  Compression), steps 3 and 5: scale = max|X|/127, code = round(X/scale); key
  observation (4) (values cluster near zero, INT8 gives a 2x ratio).
* ``kv_append`` -- "HeteroReason", workflow Phase 3 and the KVMU description
  (Fig. 7): the cache holds context plus speculated rows; rows past the
  validated length are invalid after a rejection.
* ``argmax_rows`` / ``accept_prefix`` -- "Decoding Speculative Decoding from
  First Principles", section "Speculating to get sequence parallelism during
  decode": reject at the first disagreement, keep the target's token, and the
  last row gives the +1 bonus token (1 to n+1 tokens per pass).
* ``ancestor_masks`` / ``accept_tree`` / ``commit_path`` and the
  ``draft_mask`` argument of ``spec_verify_attn`` -- the same page, section
  "Tree based verification": tree attention over each draft's lineage, the
  longest branch the target agrees with, and the surviving branch made
  contiguous in the cache.
* ``accept_stochastic`` -- the same page, section "How does this drafter
  maintain the same distribution of the target?": accept with probability
  min(1, p/q), otherwise sample the residual max(p - q, 0); random numbers
  are inputs.
* ``kvmu_apply`` -- "HeteroReason", KV Cache Management Unit (Fig. 7): the
  valid / current / step-ahead pointer triplet and its Initialization,
  Speculation, Accept and Rollback modes, plus a token-level prefix commit.
  ``reclaim_pages`` / ``alloc_pages`` -- the same section (speculative
  history discarded by pointer moves): pages wholly past the valid pointer
  return to a free list; the next step's rows take pages from it.

Pins (tests marked ``not gpu``): a torch float64 SDPA with an explicit mask and
a pure-Python triple loop for attention; closed forms (constant V rows,
identical keys, k=1 decode) and invariants (prefix invariance, page
permutation, GQA = MHA on repeated KV); a brute-force exact-rational INT8
quantiser, hand-derived tie cases and the round-trip bound; numpy.argmax and
constructed tie / NaN / signed-zero rows for acceptance; for trees, a boolean
transitive closure for the masks, torch SDPA with the tree mask, brute-force
path enumeration and chain trees reducing to the causal case; for stochastic
acceptance, the page's worked example, the output-distribution identity
located from the oracle's own decision boundaries, and the greedy limit; for
the KVMU, the page's mode table and invariants of the state machine; for the
page lists, page conservation, uniqueness and hand-worked cases.  No function here is
"parity unpinned".
"""
from .attention import spec_verify_attn
from .kv_quant import kv_quant_int8, dequant_int8, round_to_bf16
from .kv_append import kv_append
from .accept import argmax_rows, accept_prefix
from .tree import ancestor_masks, accept_tree, commit_path
from .stochastic import accept_stochastic
from .kvmu import kvmu_apply, reclaim_pages, alloc_pages

__all__ = [
    "spec_verify_attn",
    "kv_quant_int8",
    "dequant_int8",
    "round_to_bf16",
    "kv_append",
    "argmax_rows",
    "accept_prefix",
    "ancestor_masks",
    "accept_tree",
    "commit_path",
    "accept_stochastic",
    "kvmu_apply",
    "reclaim_pages",
    "alloc_pages",
]
