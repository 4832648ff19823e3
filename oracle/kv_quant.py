"""Oracle: INT8 KV quantisation with one fp16 absmax scale per (token, head) row.

Test infrastructure only (see the package docstring).

"CXL-SpecKV", Algorithm 2 (KV-Cache Compression): the scale is the absolute
maximum over the block divided by 127, and each element's code is its value
divided by that scale, rounded.  Key observation (4) motivates INT8 for KV.
Readings of what the page leaves open:

* granularity: one scale per (token, kv-head) row of d values (the algorithm
  scales a whole page; the per-row scale is the store this path exports);
* the scale is stored as fp16, rounded to nearest-even from the exact a/127;
* codes are computed against that stored fp16 scale, so dequantisation
  (code * scale) is consistent with quantisation;
* the quotient x / scale is an IEEE fp32 division, correctly rounded, and
  "round" is round-half-to-even; results are clamped to [-127, 127];
* a row whose fp16 scale is 0 (all zeros, or a/127 below half the smallest
  fp16 subnormal) gets all-zero codes.

Inputs must be finite with max|x| <= 65504 * 127, else the scale overflows.
"""
import numpy as np


def kv_quant_int8(x):
    """x [rows, d] float32 (bf16 values held in float32 are fine).

    Returns (codes [rows, d] int8, scales [rows] float16).
    """
    x32 = np.asarray(x, dtype=np.float32)
    a = np.abs(x32.astype(np.float64)).max(axis=1)            # exact
    s16 = (a / 127.0).astype(np.float16)                       # RNE to fp16
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = x32 / s16.astype(np.float32)[:, None]           # IEEE fp32 divide
    codes = np.clip(np.rint(quot), -127.0, 127.0)              # rint = half-to-even
    codes[s16 == 0] = 0.0
    return codes.astype(np.int8), s16


def dequant_int8(codes, scales):
    """codes [..., d] int8, scales [...] float16 -> float64 values (exact)."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]


def round_to_bf16(x):
    """Round float values to the nearest bfloat16 (8 significant bits), ties to
    even, returned as float64.  Covers the normal bf16 range (|x| >= 2**-126);
    zeros pass through.  Used by the append oracle for fp32 -> bf16 caches."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                                         # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)
