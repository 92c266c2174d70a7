"""Pins for the oracle's grouped quantize (CPU only).

Fixes: hand-worked rows and blocks (tests/golden), torch's IEEE fp32 division
and RNE e4m3 cast for the rowwise mode (a library routine that is independent
of the oracle's encoder), a brute-force search for the MX shared exponent and
nearest codes, power-of-two scaling invariance, and the group-coverage rule.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def h(s):
    return int(s, 16)


def bf16_of(values):
    return oracle.bf16_round_array(np.asarray(values, np.float64))


def one_group(T):
    return np.array([0, T], np.uint32)


# ----------------------------------------------------------------------------- worked examples
def test_we1_fp8_rowwise_row():
    g = GOLDEN["WE1_fp8_rowwise_row"]
    x = np.zeros((1, 32), np.uint16)
    x[0, :8] = [h(b) for b in g["x_bf16"]]
    assert np.array_equal(oracle.bf16_value_array(x[0, :8]), np.array(g["x_values"]))
    q, s = oracle.quantize(oracle.FP8_ROWWISE, x, one_group(1))
    assert [int(c) for c in q[0, :8]] == [h(c) for c in g["codes"]]
    assert np.all(q[0, 8:] == 0)
    assert s.view(np.uint32)[0] == h(g["scale_f32_bits"])


def _mx_block_case(key, fmt):
    g = GOLDEN[key]
    vals = np.zeros(32)
    vals[: len(g["x_values_then_zeros"])] = g["x_values_then_zeros"]
    x = bf16_of(vals)[None, :]
    assert np.array_equal(oracle.bf16_value_array(x[0]), vals)
    return g, oracle.quantize(fmt, x, one_group(1))


def test_we2_mxfp8_block():
    for key in ["WE2_mxfp8_block", "WE2b_mxfp8_saturating_block"]:
        g, (q, s) = _mx_block_case(key, oracle.MXFP8)
        assert s[0, 0] == h(g["scale_code"])
        n = len(g["codes_then_zeros"])
        assert [int(c) for c in q[0, :n]] == [h(c) for c in g["codes_then_zeros"]]
        assert np.all(q[0, n:] == 0)


def test_we3_mxfp4_block():
    g, (q, s) = _mx_block_case("WE3_mxfp4_block", oracle.MXFP4)
    assert s[0, 0] == h(g["scale_code"])
    n = len(g["packed_bytes_then_zeros"])
    assert [int(c) for c in q[0, :n]] == [h(c) for c in g["packed_bytes_then_zeros"]]
    assert np.all(q[0, n:] == 0)
    # nibble order: element 2i low, 2i+1 high
    nib = np.stack([q[0] & 0xF, q[0] >> 4], axis=1).ravel()
    assert [int(c) for c in nib[: len(g["nibbles_then_zeros"])]] == [h(c) for c in g["nibbles_then_zeros"]]


# ----------------------------------------------------------------------------- rowwise vs torch
def test_fp8_rowwise_matches_torch_ieee_division_and_rne_cast():
    w = W.WORKLOADS[2].scaled(tokens=16, K=1024)
    r = W.routing(w)
    x = W.activations(w, r)
    q, s = oracle.quantize(oracle.FP8_ROWWISE, W.bf16_bits(x), r.row_offsets)
    xf = x.float()
    amax = xf.abs().amax(dim=1, keepdim=True)
    scale = amax / 448.0                     # IEEE fp32 division
    v = xf / scale                           # IEEE fp32 division
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()  # RNE, |v| <= 448 here
    assert np.array_equal(s, scale.squeeze(1).numpy())
    assert np.array_equal(q, ref)


def test_fp8_rowwise_zero_row_and_subnormal_inputs():
    x = np.zeros((3, 64), np.uint16)
    x[0, 5] = 0x8000                          # -0.0 in an all-zero row
    x[1, :4] = [0x0001, 0x8001, 0x0002, 0x0000]  # bf16 subnormals only
    x[2, :2] = [0x7F7F, 0x0001]               # largest bf16 next to the smallest
    q, s = oracle.quantize(oracle.FP8_ROWWISE, x, one_group(3))
    assert s[0] == 0.0 and q[0, 5] == 0x80 and np.all(np.delete(q[0], 5) == 0)
    # row 1: amax = 2 * 2^-133 -> every element divides to +-224 or +-448
    assert q[1, 0] == oracle.e4m3_encode(224.0) and q[1, 1] == 0x80 | oracle.e4m3_encode(224.0)
    assert q[1, 2] == 0x7E
    assert q[2, 0] == 0x7E and q[2, 1] == 0x00


def test_rowwise_power_of_two_invariance():
    rng = np.random.default_rng(3)
    vals = rng.standard_normal((8, 256))
    x = bf16_of(vals)
    q0, s0 = oracle.quantize(oracle.FP8_ROWWISE, x, one_group(8))
    for j in (-5, 3, 17):
        xj = bf16_of(oracle.bf16_value_array(x) * 2.0**j)
        qj, sj = oracle.quantize(oracle.FP8_ROWWISE, xj, one_group(8))
        assert np.array_equal(qj, q0)
        assert np.array_equal(sj.astype(np.float64), s0.astype(np.float64) * 2.0**j)


# ----------------------------------------------------------------------------- MX vs brute force
def _brute_block(vals, emax, table_vals, sign_bit):
    """Shared exponent by search: the X in [-127, 127] for which amax * 2^-X
    lies in [2^emax, 2^(emax+1)) (clamped at the ends); codes by nearest
    search with ties to even and saturation."""
    amax = np.max(np.abs(vals))
    if amax == 0:
        return 0, [sign_bit if np.signbit(v) else 0 for v in vals]
    X = None
    for cand in range(-127, 128):
        m = amax * 2.0 ** (-cand)
        if 2.0**emax <= m < 2.0 ** (emax + 1):
            X = cand
    if X is None:
        X = -127 if amax * 2.0**127 < 2.0**emax else 127
    codes = []
    for v in vals:
        a = abs(v) * 2.0 ** (-X)
        d = np.abs(table_vals - a)
        best = np.nonzero(d == d.min())[0]
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        if a >= table_vals[-1]:
            c = len(table_vals) - 1
        codes.append(c | (sign_bit if np.signbit(v) else 0))
    return X + 127, codes


def test_mx_quantize_brute_force_blocks():
    rng = np.random.default_rng(5)
    e4m3_tab = oracle.e4m3_value_array(np.arange(0x7F, dtype=np.uint8))
    e2m1_tab = np.array(GOLDEN["e2m1_values"]["codes_0_to_7"])
    blocks = [rng.standard_normal(32) * 10.0 ** rng.integers(-38, 38) for _ in range(60)]
    blocks.append(np.zeros(32))
    blocks.append(np.r_[-0.0, np.zeros(31)])
    blocks.append(np.r_[2.0**-133, -(2.0**-133), np.zeros(30)])   # bf16 subnormals
    blocks.append(np.r_[3.3895313892515355e38, 1.0, np.zeros(30)])
    x = bf16_of(np.stack(blocks))
    vals = oracle.bf16_value_array(x)
    q8, s8 = oracle.quantize(oracle.MXFP8, x, one_group(len(blocks)))
    q4, s4 = oracle.quantize(oracle.MXFP4, x, one_group(len(blocks)))
    for i, v in enumerate(vals):
        sc, codes = _brute_block(v, 8, e4m3_tab, 0x80)
        assert s8[i, 0] == sc and list(q8[i]) == codes, i
        sc, codes = _brute_block(v, 2, e2m1_tab, 0x8)
        nib = np.stack([q4[i] & 0xF, q4[i] >> 4], axis=1).ravel()
        assert s4[i, 0] == sc and list(nib) == codes, i


def test_mx_power_of_two_invariance():
    rng = np.random.default_rng(9)
    x = bf16_of(rng.standard_normal((4, 128)))
    for fmt in (oracle.MXFP8, oracle.MXFP4):
        q0, s0 = oracle.quantize(fmt, x, one_group(4))
        for j in (-9, 4):
            xj = bf16_of(oracle.bf16_value_array(x) * 2.0**j)
            qj, sj = oracle.quantize(fmt, xj, one_group(4))
            assert np.array_equal(qj, q0)
            assert np.array_equal(sj.astype(int), s0.astype(int) + j)


# ----------------------------------------------------------------------------- group coverage
def test_quantize_only_touches_grouped_rows():
    rng = np.random.default_rng(1)
    x = bf16_of(rng.standard_normal((10, 64)))
    off = np.array([2, 2, 5, 5, 8], np.uint32)  # rows 2..7 in groups 1 and 3; 0,1,8,9 uncovered
    for fmt in (oracle.FP8_ROWWISE, oracle.MXFP8, oracle.MXFP4):
        qcols = 32 if fmt == oracle.MXFP4 else 64
        q = np.full((10, qcols), 0xA5, np.uint8)
        s = np.full((10,), -7.0, np.float32) if fmt == 0 else np.full((10, 2), 0x5A, np.uint8)
        q, s = oracle.quantize(fmt, x, off, q, s)
        qa, sa = oracle.quantize(fmt, x, one_group(10))
        for t in range(10):
            if 2 <= t < 8:
                assert np.array_equal(q[t], qa[t]) and np.array_equal(s[t], sa[t])
            else:
                assert np.all(q[t] == 0xA5) and np.all(s[t] == (-7.0 if fmt == 0 else 0x5A))


def test_quantize_clamps_offsets_and_skips_inverted_groups():
    rng = np.random.default_rng(2)
    x = bf16_of(rng.standard_normal((6, 32)))
    off = np.array([4, 1, 3, 100], np.uint32)  # g0 inverted (skipped), g1 = [1,3), g2 = [3, 6) clamped
    q = np.full((6, 32), 0xA5, np.uint8)
    s = np.full((6,), -1.0, np.float32)
    q, s = oracle.quantize(oracle.FP8_ROWWISE, x, off, q, s)
    qa, sa = oracle.quantize(oracle.FP8_ROWWISE, x, one_group(6))
    assert np.all(q[0] == 0xA5) and s[0] == -1.0
    assert np.array_equal(q[1:], qa[1:]) and np.array_equal(s[1:], sa[1:])


# ---------------------------------------------------------------- gathered quantize
# (NvMxf4f8Strategy, grouped_quantize(): indices / indices_divisor.  Reading:
#  routed row t is source row indices[t] // indices_divisor.)  The gathered
# form must equal the pinned plain quantize of the rows it names, and rows
# whose index names no source row must keep their contents.
@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_quantize_gather_identity_equals_quantize(fmt):
    rng = np.random.default_rng(40 + fmt)
    T, K = 37, 96
    x = oracle.bf16_round_array(rng.standard_normal((T, K)) * np.exp(rng.uniform(-4, 4, (T, 1))))
    off = np.array([0, 10, 10, 30, T], np.uint32)
    q0, s0 = oracle.quantize(fmt, x, off)
    q1, s1 = oracle.quantize_gather(fmt, x, np.arange(T, dtype=np.int32), 1, off)
    assert np.array_equal(q0, q1) and np.array_equal(s0.view(np.uint8), s1.view(np.uint8))


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_quantize_gather_follows_indices_and_divisor(fmt):
    rng = np.random.default_rng(50 + fmt)
    S, top_k, K = 23, 4, 64
    x = oracle.bf16_round_array(rng.standard_normal((S, K)))
    # every (token, k) slot once, sorted by a random expert -> routed rows
    slots = rng.permutation(S * top_k).astype(np.int32)
    T = slots.size
    off = np.array([0, 30, 31, 60, T], np.uint32)
    q, s = oracle.quantize_gather(fmt, x, slots, top_k, off)
    qr, sr = oracle.quantize(fmt, x[slots // top_k], off)
    assert np.array_equal(q, qr) and np.array_equal(s.view(np.uint8), sr.view(np.uint8))


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_quantize_gather_skips_rows_without_a_source(fmt):
    rng = np.random.default_rng(60 + fmt)
    S, K = 5, 32
    x = oracle.bf16_round_array(rng.standard_normal((S, K)))
    idx = np.array([0, -1, 9, 10, 4, 2**31 - 1, 7], np.int32)  # divisor 2: sources 0, -, 4, 5(out), 2, out, 3
    T = idx.size
    off = np.array([0, T], np.uint32)
    qcols = K // 2 if fmt == 2 else K
    q0 = np.full((T, qcols), 0xA5, np.uint8)
    s0 = np.full((T,), -3.0, np.float32) if fmt == 0 else np.full((T, K // 32), 0x5A, np.uint8)
    q, s = oracle.quantize_gather(fmt, x, idx, 2, off, q0.copy(), s0.copy())
    for t, v in enumerate(idx):
        src = v // 2
        if v < 0 or src >= S:
            assert np.all(q[t] == 0xA5) and np.array_equal(np.atleast_1d(s[t]).view(np.uint8),
                                                           np.atleast_1d(s0[t]).view(np.uint8))
        else:
            qr, sr = oracle.quantize(fmt, x[src:src + 1], np.array([0, 1], np.uint32))
            assert np.array_equal(q[t], qr[0]) and np.array_equal(np.atleast_1d(s[t]).view(np.uint8),
                                                                  np.atleast_1d(sr[0]).view(np.uint8))


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_quantize_scatter_equals_quantize_of_the_routed_rows(fmt):
    """Token-major form: routed rows named through the inverse slot map get
    exactly the quantization of their token row, as if the routed rows had
    been materialised and quantized (every slot of every token routed once)."""
    rng = np.random.default_rng(70 + fmt)
    S, top_k, K = 19, 4, 96
    x = oracle.bf16_round_array(rng.standard_normal((S, K)) * np.exp(rng.uniform(-6, 6, (S, 1))))
    slots = rng.permutation(S * top_k).astype(np.int32)   # routed row t serves slot slots[t]
    T = slots.size
    ros = np.empty(T, np.int32)
    ros[slots] = np.arange(T, dtype=np.int32)              # the inverse map
    off = np.array([0, 20, 20, 51, T], np.uint32)
    q, s = oracle.quantize_scatter(fmt, x, ros, T, off)
    qr, sr = oracle.quantize(fmt, x[slots // top_k], off)
    assert np.array_equal(q, qr) and np.array_equal(s.view(np.uint8), sr.view(np.uint8))
    qg, sg = oracle.quantize_gather(fmt, x, slots, top_k, off)
    assert np.array_equal(q, qg) and np.array_equal(s.view(np.uint8), sg.view(np.uint8))


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_quantize_scatter_leaves_dropped_and_uncovered_rows(fmt):
    rng = np.random.default_rng(80 + fmt)
    S, top_k, K, T = 6, 2, 64, 14
    x = oracle.bf16_round_array(rng.standard_normal((S, K)))
    ros = np.array([0, 13, -1, 5, 20, 7, 3, 2**31 - 1, 9, 11, 12, -5], np.int32)
    off = np.array([2, 5, 3, 7, 12], np.uint32)         # rows 2..11 covered (g1 inverted, g2 overlaps g0)
    qcols = K // 2 if fmt == 2 else K
    q0 = np.full((T, qcols), 0xA5, np.uint8)
    s0 = np.full((T,), -3.0, np.float32) if fmt == 0 else np.full((T, K // 32), 0x5A, np.uint8)
    q, s = oracle.quantize_scatter(fmt, x, ros, T, off, q0.copy(), s0.copy())
    written = {}
    for i, r in enumerate(ros):
        if 2 <= r < 12:
            written[int(r)] = i // top_k
    for r in range(T):
        if r in written:
            qr, sr = oracle.quantize(fmt, x[written[r]:written[r] + 1], np.array([0, 1], np.uint32))
            assert np.array_equal(q[r], qr[0]) and np.array_equal(np.atleast_1d(s[r]).view(np.uint8),
                                                                  np.atleast_1d(sr[0]).view(np.uint8)), r
        else:
            assert np.all(q[r] == 0xA5) and np.array_equal(np.atleast_1d(s[r]).view(np.uint8),
                                                           np.atleast_1d(s0[r]).view(np.uint8)), r
    assert set(written) == {3, 5, 7, 9, 11}
