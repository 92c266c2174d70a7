"""Pins for the oracle's element codecs (CPU only).

Each check fixes the oracle against something other than its own formulas:
published code tables (OCP OFP8 / OCP MX v1.0), torch's independent fp8 / e8m0
decoders and RNE casts, brute-force nearest-code search over every code, and
hand-worked examples stored under tests/golden/.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def h(s):
    return int(s, 16)


# ----------------------------------------------------------------------------- decoders
def test_e4m3_decode_matches_torch_for_all_256_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_value_array(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_landmarks():
    g = GOLDEN["e4m3_landmarks"]
    for code, val in g["values"].items():
        v = oracle.e4m3_value(h(code))
        assert v == val and np.signbit(v) == np.signbit(val), code
    for code in g["nan_codes"]:
        assert np.isnan(oracle.e4m3_value(h(code)))


def test_e4m3_positive_codes_are_strictly_increasing():
    v = oracle.e4m3_value_array(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    # negative half mirrors the positive half
    n = oracle.e4m3_value_array(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(n, -v)


def test_e2m1_decode_matches_ocp_table():
    table = GOLDEN["e2m1_values"]["codes_0_to_7"]
    for c in range(8):
        assert oracle.e2m1_value(c) == table[c]
        assert oracle.e2m1_value(c | 8) == -table[c]
    assert np.signbit(oracle.e2m1_value(8))


def test_e8m0_decode_matches_torch_for_all_256_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().double().numpy()
    for c in range(256):
        v = oracle.e8m0_value(c)
        if c == 255:
            assert np.isnan(v) and np.isnan(ref[c])
        else:
            assert v == 2.0 ** (c - 127) == ref[c]


def test_bf16_decode_is_the_high_half_of_binary32():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    for b in [0x0000, 0x8000, 0x3F80, 0x0001, 0x7F7F, 0xFF7F, 0x4060, 0x3DCD]:
        assert oracle.bf16_value(b) == ref[b]


# ----------------------------------------------------------------------------- encoders
def _finite_bf16_values():
    bits = np.arange(65536, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return vals[np.isfinite(vals)]


def _brute_nearest(values, code_vals, max_code):
    """Nearest finite non-negative code (index into code_vals) for |value|: a
    tie between two nearest codes goes to the even code (even mantissa bit);
    magnitudes at or above the largest code saturate to it."""
    codes = np.arange(code_vals.size)
    a = np.abs(values)
    d = np.abs(a[:, None] - code_vals[None, :])
    is_best = d == d.min(axis=1, keepdims=True)
    n_best = is_best.sum(axis=1)
    first = np.argmax(is_best, axis=1)
    even_pick = np.where(is_best & (codes[None, :] % 2 == 0), codes[None, :], 10**6).min(axis=1)
    mag = np.where(n_best > 1, even_pick, codes[first])
    return np.where(a >= code_vals[max_code], max_code, mag)


def test_e4m3_encode_brute_force_all_bf16():
    vals = _finite_bf16_values()
    ours = oracle.e4m3_encode_array(vals)
    cvals = oracle.e4m3_value_array(np.arange(0x7F, dtype=np.uint8))  # 0x00 .. 0x7e
    mag = _brute_nearest(vals, cvals, 0x7E)
    expect = (mag | np.where(np.signbit(vals), 0x80, 0)).astype(np.uint8)
    assert np.array_equal(ours, expect)


def test_e4m3_encode_matches_torch_cast_in_range():
    vals = _finite_bf16_values()
    vals = vals[np.abs(vals) < 448.0]
    ours = oracle.e4m3_encode_array(vals)
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e2m1_encode_brute_force_all_bf16():
    vals = _finite_bf16_values()
    ours = oracle.e2m1_encode_array(vals)
    cvals = np.array(GOLDEN["e2m1_values"]["codes_0_to_7"])
    mag = _brute_nearest(vals, cvals, 7)
    expect = (mag | np.where(np.signbit(vals), 8, 0)).astype(np.uint8)
    assert np.array_equal(ours, expect)


def test_e4m3_encode_worked_cases():
    for v, code in GOLDEN["e4m3_encode"]["cases"]:
        assert oracle.e4m3_encode(v) == h(code), (v, code)


def test_e2m1_encode_worked_cases():
    for v, code in GOLDEN["e2m1_encode"]["cases"]:
        assert oracle.e2m1_encode(v) == h(code), (v, code)


def test_encode_decode_round_trip_all_codes():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c
    for c in range(16):
        assert oracle.e2m1_encode(oracle.e2m1_value(c)) == c


# ----------------------------------------------------------------------------- bf16 rounding
def _bf16_nearest_exact(v: float) -> int:
    """Exact-rational nearest bf16 (ties to even bit pattern), for finite v in range."""
    f = Fraction(v)
    a = abs(f)
    lo = int(np.float32(float(a)).view(np.uint32) >> 16)  # a candidate near a
    best = None
    for bits in range(max(lo - 2, 0), min(lo + 3, 0x7F80)):
        val = Fraction(float((np.uint32(bits) << np.uint32(16)).view(np.float32)))
        d = abs(val - a)
        key = (d, bits % 2)
        if best is None or key < best[0]:
            best = (key, bits)
    sign = 0x8000 if np.signbit(v) else 0
    return sign | best[1]


def test_bf16_round_against_exact_rational_search():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    # midpoints and near-midpoints between neighbouring bf16 values
    for bits in rng.integers(0x0080, 0x7F00, 500):
        lo = float((np.uint32(bits) << np.uint32(16)).view(np.float32))
        hi = float((np.uint32(bits + 1) << np.uint32(16)).view(np.float32))
        mid = (lo + hi) / 2
        vals += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf), -mid]
    for v in vals:
        assert oracle.bf16_round(v) == _bf16_nearest_exact(v), v


def test_bf16_round_worked_cases():
    for v, bits in GOLDEN["bf16_round"]["cases"]:
        assert oracle.bf16_round(v) == h(bits), (v, bits)


def test_bf16_round_avoids_double_rounding():
    # 1 + 2^-8 + 2^-30 lies just above a bf16 tie; going through fp32 first
    # would land exactly on the tie and round down to 1.0.
    v = 1.0 + 2.0**-8 + 2.0**-30
    assert oracle.bf16_round(v) == 0x3F81
    assert oracle.bf16_round(float(np.float32(v))) == 0x3F80


def test_bf16_round_agrees_with_torch_on_fp32_representable_values():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    ours = oracle.bf16_round_array(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
