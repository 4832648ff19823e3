"""Pins for the INT8 quantisation oracle (CPU only).

"CXL-SpecKV", Algorithm 2: scale = max|X|/127, code = round(X/scale).  The
pins are an exact-rational brute force (every fp16 value enumerated, the fp32
quotient rounded by neighbour search, Python's half-to-even round), tie cases
derived by hand, the round-trip bound, symmetry, idempotence, and the
page's 2.00x INT8 ratio as a closed form (tests/golden/int8_ratio.txt).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

_F16_ALL = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)     # +0 .. max finite
_F16_FR = [Fraction(float(v)) for v in _F16_ALL]


def _round_fraction_to_f16(r):
    """Nearest non-negative fp16 to the rational r, ties to even (brute force)."""
    best = None
    for idx, v in enumerate(_F16_FR):
        dist = abs(v - r)
        if best is None or dist < best[0] or (dist == best[0] and idx % 2 == 0):
            best = (dist, idx)
    return _F16_ALL[best[1]]


def _round_fraction_to_f32(r):
    """Nearest fp32 to rational r, ties to even, by neighbour search."""
    f = np.float32(float(r))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        dist = abs(Fraction(float(c)) - r)
        even = (np.array(c, np.float32).view(np.uint32) & 1) == 0
        if best is None or dist < best[0] or (dist == best[0] and even):
            best = (dist, c)
    return best[1]


def _brute_quant(row):
    a = max(abs(Fraction(float(x))) for x in row)
    s16 = _round_fraction_to_f16(a / 127)
    if s16 == 0:
        return [0] * len(row), s16
    codes = []
    for x in row:
        qf = _round_fraction_to_f32(Fraction(float(x)) / Fraction(float(s16)))
        c = round(Fraction(float(qf)))           # Python rounds halves to even
        codes.append(max(-127, min(127, c)))
    return codes, s16


def test_matches_exact_rational_brute_force():
    rng = np.random.default_rng(3)
    rows = [rng.standard_normal(8).astype(np.float32) * s for s in (1.0, 0.5, 1e-3, 37.0, 1e-6)]
    rows.append(np.array([31.75, 0.125, 0.375, 0.625, -0.125, -0.375, -0.625, 0.0], np.float32))
    rows.append(np.zeros(8, np.float32))
    rows.append(np.array([1e-9, -2e-9, 0, 0, 0, 0, 0, 5e-10], np.float32))   # fp16 scale underflows
    rows.append(np.array([3.0e6, -1.0, 2.5, 0, 7.0, -3.0e6, 1e5, 8.0], np.float32))
    x = np.stack(rows)
    codes, scales = oracle.kv_quant_int8(x)
    for r, row in enumerate(x):
        bc, bs = _brute_quant(row)
        assert scales[r].view(np.uint16) == np.float16(bs).view(np.uint16), r
        assert list(codes[r]) == bc, r


def test_hand_derived_ties():
    # 31.75 / 127 = 0.25 exactly, so the fp16 scale is 0.25 and x / 0.25 lands on
    # exact halves 0.5, 1.5, 2.5 -> 0, 2, 2 under half-to-even.
    x = np.array([[31.75, 0.125, 0.375, 0.625, -0.125, -0.375, -0.625,
                   np.nextafter(np.float32(0.125), np.float32(1)),
                   np.nextafter(np.float32(0.375), np.float32(0))]], np.float32)
    codes, s = oracle.kv_quant_int8(x)
    assert float(s[0]) == 0.25
    assert list(codes[0]) == [127, 0, 2, 2, 0, -2, -2, 1, 1]


def test_round_trip_bound_absmax_and_symmetry():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((200, 64)) * rng.uniform(1e-3, 10, (200, 1))).astype(np.float32)
    codes, s = oracle.kv_quant_int8(x)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * s64)
    assert (err <= s64 * (0.5 + 2.0 ** -17)).all()
    am = np.abs(x).argmax(axis=1)
    assert (np.abs(codes[np.arange(200), am]) == 127).all()
    assert (codes >= -127).all() and (codes <= 127).all()
    c2, s2 = oracle.kv_quant_int8(-x)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, s)


def test_idempotent_on_dequantised_values():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((100, 128)).astype(np.float32) * 0.5
    codes, s = oracle.kv_quant_int8(x)
    y = oracle.dequant_int8(codes, s)
    assert np.array_equal(y.astype(np.float32).astype(np.float64), y)    # exact in fp32
    c2, s2 = oracle.kv_quant_int8(y.astype(np.float32))
    assert np.array_equal(c2, codes) and np.array_equal(s2, s)


def test_zero_row():
    codes, s = oracle.kv_quant_int8(np.zeros((2, 16), np.float32))
    assert (codes == 0).all() and (s == 0).all()


def _golden(name):
    vals = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                vals[k.strip()] = float(v)
    return vals


def test_int8_bytes_ratio_closed_form():
    g = _golden("int8_ratio.txt")
    d = 128
    x = np.random.default_rng(6).standard_normal((16, d)).astype(np.float32)
    codes, s = oracle.kv_quant_int8(x)
    bf16_bytes = x.size * 2
    per_row = bf16_bytes / (codes.nbytes + s.nbytes)            # one fp16 scale per row
    assert per_row == pytest.approx(2 * d / (d + 2))
    assert per_row == pytest.approx(g["per_row_ratio_d128"], abs=5e-4)
    per_page = bf16_bytes / (codes.nbytes + 2)                  # one scale per 16-row page
    assert per_page == pytest.approx(g["per_page_ratio_d128"], abs=5e-4)
    assert round(per_page, 2) == g["page_int8_only_ratio"]


def test_round_to_bf16_matches_torch_conversion():
    import torch
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                        [0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_bf16(x), ref)
