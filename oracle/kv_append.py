"""Oracle: append the k_b new K/V rows of each sequence into its paged cache.

Test infrastructure only (see the package docstring).

"HeteroReason", workflow Phase 3 and the KVMU description (Fig. 7): during
speculation the cache holds the validated context followed by the speculated
rows; after acceptance the valid pointer simply moves forward, and after a
rejection the rows past it are invalid.  Here draft row i of sequence b is
written at logical position S_b + i, i.e. physical page
block_table[b][(S_b+i) // page], slot (S_b+i) % page.  An INT8 cache stores
the row quantised with ``kv_quant_int8``; a bf16 cache stores the row rounded
to nearest-even bf16; an fp32 cache stores it unchanged.
"""
import numpy as np

from .kv_quant import kv_quant_int8, round_to_bf16


def kv_append(k_new, v_new, k_pool, v_pool, block_table, ctx_lens, cu_q, cache_dtype,
              k_scale=None, v_scale=None):
    """Returns updated copies (k_pool, v_pool, k_scale, v_scale).

    k_new/v_new [T, Hkv, d] float; pools [P, Hkv, page, d] (float64 values for
    float caches, int8 codes for 'int8' with float16 scales [P, Hkv, page]).
    cache_dtype in {'f32', 'bf16', 'int8'}.
    """
    k_pool = np.array(k_pool, copy=True)
    v_pool = np.array(v_pool, copy=True)
    if cache_dtype == "int8":
        k_scale = np.array(k_scale, copy=True)
        v_scale = np.array(v_scale, copy=True)
    page = k_pool.shape[2]
    B = len(ctx_lens)
    for b in range(B):
        S = int(ctx_lens[b])
        for t in range(int(cu_q[b]), int(cu_q[b + 1])):
            pos = S + (t - int(cu_q[b]))
            pg = int(block_table[b][pos // page])
            sl = pos % page
            for src, pool, scl in ((k_new, k_pool, k_scale), (v_new, v_pool, v_scale)):
                row = np.asarray(src[t], dtype=np.float32)     # [Hkv, d]
                if cache_dtype == "int8":
                    codes, s16 = kv_quant_int8(row)
                    pool[pg, :, sl, :] = codes
                    scl[pg, :, sl] = s16
                elif cache_dtype == "bf16":
                    pool[pg, :, sl, :] = round_to_bf16(row)
                else:
                    pool[pg, :, sl, :] = row.astype(np.float64)
    return k_pool, v_pool, k_scale, v_scale
