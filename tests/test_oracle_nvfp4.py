"""Pins for the oracle's NVFP4 quantize and grouped GEMM (CPU only).

The pages name NVFP4 (16-element blocks with E4M3 block scales and a
per-expert tensor scale) without its arithmetic; the readings are stated in
oracle.c.  Fixes: hand-worked blocks and a 1x1 GEMM (tests/golden), the
special blocks (zero, underflow, saturation), block locality (16 elements per
scale), invariance of codes when x and the tensor scale trade a power of two
(catches a tensor scale applied the wrong way round), the GEMM against a
numpy matmul of independently decoded operands, and the GEMM against the
already pinned MXFP4 oracle where every NVFP4 block scale is 1.  The
SwiGLU + NVFP4 requant is pinned as the NVFP4 quantize of the pinned MXFP4
path's y, the fused rows as that requant of the pinned NVFP4 GEMM, and the
row scale by trading a power of two with the expert scale.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def h(s):
    return int(s, 16)


def bf16_of(values):
    return oracle.bf16_round_array(np.asarray(values, np.float64))


def one_group(T):
    return np.array([0, T], np.uint32), np.zeros(1, np.int32)


# Independent decoders (table and bit fields written out here, not the oracle's).
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)


def e4m3_decode(codes):
    c = np.asarray(codes, np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * 2.0 ** (e - 7))
    return sign * val


def unpack_fp4(q):
    q = np.asarray(q, np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


@pytest.mark.parametrize("key", ["WE7_nvfp4_block", "WE7b_nvfp4_scaled_block"])
def test_worked_blocks(key):
    g = GOLDEN[key]
    x = bf16_of(g["x_values"]).reshape(1, 16)
    off, ids = one_group(1)
    q, s = oracle.quantize_nvfp4(x, off, ids, [g["sf"]])
    assert int(s[0, 0]) == h(g["scale_code"])
    assert [int(c) for c in unpack_fp4(q)[0]] == [h(c) for c in g["nibbles"]]
    assert [int(b) for b in q[0]] == [h(b) for b in g["packed_bytes"]]


def test_worked_gemm_1x1():
    g = GOLDEN["WE8_nvfp4_gemm_1x1"]
    we7 = GOLDEN["WE7_nvfp4_block"]
    a = np.array([[h(b) for b in we7["packed_bytes"]]], np.uint8)
    sa = np.array([[h(we7["scale_code"])]], np.uint8)
    b = np.full((1, 1, 8), 0x22, np.uint8)
    sb = np.full((1, 1, 1), 0x3C, np.uint8)
    off, ids = one_group(1)
    r = oracle.gemm_rows_nvfp4(a, sa, b, sb, [g["expert_scale"]], off, ids, 1, 16, [0])
    assert r["exact"][0, 0] == 11.25
    assert int(r["out"][0, 0]) == h(g["out_bf16"])


def test_special_blocks():
    off, ids = one_group(1)
    # all zero (with a negative zero): scale 0, signed-zero codes
    x = bf16_of([0.0] * 15 + [-0.0]).reshape(1, 16)
    q, s = oracle.quantize_nvfp4(x, off, ids, [3.0])
    assert s[0, 0] == 0 and list(unpack_fp4(q)[0]) == [0] * 15 + [8]
    # underflow: amax/6*sf below half the smallest E4M3 subnormal (2^-10) -> scale 0, codes zero
    x = bf16_of([2.0 ** -12, -(2.0 ** -12)] + [0.0] * 14).reshape(1, 16)
    q, s = oracle.quantize_nvfp4(x, off, ids, [1.0])
    assert s[0, 0] == 0 and list(unpack_fp4(q)[0][:2]) == [0, 8]
    # saturation of the block scale: amax/6*sf > 448 -> 0x7e (448), elements x*sf/448
    x = bf16_of([600.0, 300.0, -150.0] + [0.0] * 13).reshape(1, 16)
    q, s = oracle.quantize_nvfp4(x, off, ids, [6.0])
    assert s[0, 0] == 0x7E
    # 600*6/448 = 8.04 -> 6 (code 7); 300*6/448 = 4.02 -> 4 (code 6); -150*6/448 = -2.01 -> -2 (code 0xc)
    assert list(unpack_fp4(q)[0][:3]) == [0x7, 0x6, 0xC]


def test_sixteen_element_blocks():
    rng = np.random.default_rng(7)
    x = bf16_of(rng.normal(size=(1, 64))).reshape(1, 64)
    off, ids = one_group(1)
    q0, s0 = oracle.quantize_nvfp4(x, off, ids, [10.0])
    assert s0.shape == (1, 4) and q0.shape == (1, 32)
    x2 = x.copy()
    x2[0, 20] = bf16_of([40.0])[0]  # a new amax inside the second 16-block only
    q1, s1 = oracle.quantize_nvfp4(x2, off, ids, [10.0])
    assert s1[0, 1] != s0[0, 1]
    assert s1[0, 0] == s0[0, 0] and s1[0, 2] == s0[0, 2] and s1[0, 3] == s0[0, 3]
    assert np.array_equal(q1[0, :8], q0[0, :8]) and np.array_equal(q1[0, 16:], q0[0, 16:])


@pytest.mark.parametrize("j", [-3, 2, 5])
def test_power_of_two_trade(j):
    """x * 2^j with sf * 2^-j gives the same codes and scales (all steps exact
    under power-of-two scaling away from underflow and saturation); a tensor
    scale applied as a divisor instead would break this."""
    rng = np.random.default_rng(11)
    x = bf16_of(rng.normal(size=(8, 64)) * 3.0)
    xs = bf16_of(oracle.bf16_value_array(x) * 2.0 ** j)
    off, ids = one_group(8)
    sf = 37.0
    q0, s0 = oracle.quantize_nvfp4(x, off, ids, [sf])
    q1, s1 = oracle.quantize_nvfp4(xs, off, ids, [sf * 2.0 ** -j])
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)
    # and the dequantized row tracks x: |x - q*s/sf| <= amax_block / 6 + its e4m3 rounding
    xv = oracle.bf16_value_array(x).reshape(8, 4, 16)
    deq = (E2M1[unpack_fp4(q0)].reshape(8, 4, 16) * e4m3_decode(s0)[..., None]) / sf
    amax = np.abs(xv).max(axis=2, keepdims=True)
    assert np.all(np.abs(xv - deq) <= amax * (1.0 / 6 + 1.0 / 16) + 1e-12)


def test_groups_use_their_expert_tensor_scale():
    rng = np.random.default_rng(3)
    x = bf16_of(rng.normal(size=(10, 32)))
    off = np.array([0, 4, 4, 10], np.uint32)
    ids = np.array([2, 0, 1], np.int32)
    sf = np.array([1.0, 5.0, 20.0], np.float32)
    q, s = oracle.quantize_nvfp4(x, off, ids, sf)
    for rows, e in [(range(0, 4), 2), (range(4, 10), 1)]:
        for t in rows:
            qe, se = oracle.quantize_nvfp4(x[t:t + 1], np.array([0, 1], np.uint32), np.zeros(1, np.int32), [sf[e]])
            assert np.array_equal(q[t], qe[0]) and np.array_equal(s[t], se[0])
    # an expert id outside [0, E) skips its group: the rows keep their contents
    q2 = np.full((10, 16), 0x5A, np.uint8)
    s2 = np.full((10, 2), 0xA5, np.uint8)
    oracle.quantize_nvfp4(x, np.array([0, 10], np.uint32), np.array([3], np.int32), sf, q2, s2)
    assert np.all(q2 == 0x5A) and np.all(s2 == 0xA5)


def random_nvfp4(rng, shape_rows, K):
    q = rng.integers(0, 256, size=shape_rows + (K // 2,), dtype=np.uint8)
    s = rng.integers(0x20, 0x50, size=shape_rows + (K // 16,), dtype=np.uint8)  # E4M3 2^-4 .. 2^2 range
    return q, s


def test_gemm_equals_matmul_of_decoded_operands():
    rng = np.random.default_rng(5)
    E, N, K = 3, 24, 96
    off = np.array([0, 5, 5, 13], np.uint32)
    ids = np.array([2, 0, 1], np.int32)
    a, sa = random_nvfp4(rng, (13,), K)
    b, sb = random_nvfp4(rng, (E, N), K)
    es = np.array([0.5, 2.0, 0.125], np.float32)
    r = oracle.gemm_rows_nvfp4(a, sa, b, sb, es, off, ids, N, K, np.arange(13))
    A = E2M1[unpack_fp4(a)] * np.repeat(e4m3_decode(sa), 16, axis=1)
    B = E2M1[unpack_fp4(b)] * np.repeat(e4m3_decode(sb), 16, axis=2)
    for t in range(13):
        g = 0 if t < 5 else 2
        e = ids[g]
        ref = (A[t] @ B[e].T) * float(es[e])
        assert r["group"][t] == g
        np.testing.assert_allclose(r["exact"][t], ref, rtol=1e-12, atol=1e-12)


def test_gemm_with_unit_block_scales_equals_mxfp4():
    """All NVFP4 block scales 0x38 (1.0), expert scale 1: the MXFP4 oracle with
    E8M0 scale 127 (1.0) on the same codes must give the same result."""
    rng = np.random.default_rng(9)
    E, N, K = 2, 16, 128
    off = np.array([0, 6, 11], np.uint32)
    ids = np.array([1, 0], np.int32)
    a = rng.integers(0, 256, size=(11, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    nv = oracle.gemm_rows_nvfp4(a, np.full((11, K // 16), 0x38, np.uint8), b, np.full((E, N, K // 16), 0x38, np.uint8),
                                np.ones(E, np.float32), off, ids, N, K, np.arange(11))
    mx = oracle.gemm_rows(oracle.MXFP4, a, np.full((11, K // 32), 127, np.uint8), b,
                          np.full((E, N, K // 32), 127, np.uint8), off, ids, N, K, np.arange(11))
    assert np.array_equal(nv["exact"], mx["exact"]) and np.array_equal(nv["out"], mx["out"])


# ----------------------------------------------------------------------------- SwiGLU + NVFP4 requant
def gate_up(rng, T, I):
    vals = rng.standard_normal((T, 2 * I)) * np.exp(rng.uniform(-4, 3, (T, 1)))
    vals[0, :6] = [0.0, 5.0, 20.0, 0.25, -0.0, 3.0]
    return oracle.bf16_round_array(vals)


def test_silu_requant_nvfp4_is_the_nvfp4_quantize_of_y():
    """The requant is the (pinned) NVFP4 quantize applied to y = bf16(silu(g) u),
    with y taken from the (pinned) MXFP4 requant's fp64 y."""
    rng = np.random.default_rng(17)
    T, I = 9, 64
    h = gate_up(rng, T, I)
    off = np.array([0, 4, 9], np.uint32)
    ids = np.array([1, 0], np.int32)
    sf = np.array([3.0, 250.0], np.float32)
    yq, ys = oracle.silu_requant_nvfp4(h, off, ids, sf)
    _, _, y64 = oracle.silu_requant(h, np.array([0, T], np.uint32), want_y64=True)
    yb = oracle.bf16_round_array(y64)
    q_ref, s_ref = oracle.quantize_nvfp4(yb, off, ids, sf)
    assert np.array_equal(yq, q_ref) and np.array_equal(ys, s_ref)
    # g = 20, u = 0.25: silu(20) * 0.25 rounds to 5.0 exactly; g = 0 gives 0
    assert oracle.bf16_value_array(yb[0, :3]).tolist() == [0.0, 5.0, 0.0]


def test_gemm_swiglu_nvfp4_composes_gemm_and_requant():
    rng = np.random.default_rng(23)
    E, I, K = 3, 32, 64
    off = np.array([0, 4, 4, 10], np.uint32)
    ids = np.array([2, 0, 1], np.int32)
    a, sa = random_nvfp4(rng, (10,), K)
    w, ws = random_nvfp4(rng, (E, 2 * I), K)
    es = np.array([0.5, 0.25, 1.0], np.float32)
    rs = oracle.bf16_round_array(rng.uniform(0.5, 2.0, 10))
    sfy = np.array([10.0, 2.0, 40.0], np.float32)
    rows = np.arange(10)
    fused = oracle.gemm_swiglu_rows_nvfp4(a, sa, w, ws, es, rs, sfy, off, ids, I, K, rows)
    g = oracle.gemm_rows_nvfp4(a, sa, w, ws, es, off, ids, 2 * I, K, rows)
    h = oracle.bf16_round_array(g["exact"] * oracle.bf16_value_array(rs)[:, None])
    yq, ys = oracle.silu_requant_nvfp4(h, off, ids, sfy)
    cov = fused["group"] >= 0
    assert np.array_equal(fused["yq"][cov], yq[cov]) and np.array_equal(fused["ys"][cov], ys[cov])
    np.testing.assert_array_equal(fused["gu_exact"][cov], (g["exact"] * oracle.bf16_value_array(rs)[:, None])[cov])


def test_gemm_swiglu_nvfp4_row_scale_trades_with_expert_scale():
    """Row scale 2^j with expert scale 2^-j leaves every output unchanged (all
    products exact); no row scale is the row scale 1."""
    rng = np.random.default_rng(29)
    E, I, K = 2, 32, 32
    off = np.array([0, 5, 8], np.uint32)
    ids = np.array([0, 1], np.int32)
    a, sa = random_nvfp4(rng, (8,), K)
    w, ws = random_nvfp4(rng, (E, 2 * I), K)
    sfy = np.array([5.0, 7.0], np.float32)
    es = np.array([1.0, 0.5], np.float32)
    base = oracle.gemm_swiglu_rows_nvfp4(a, sa, w, ws, es, None, sfy, off, ids, I, K, np.arange(8))
    rs = oracle.bf16_round_array(np.full(8, 4.0))
    traded = oracle.gemm_swiglu_rows_nvfp4(a, sa, w, ws, es / 4, rs, sfy, off, ids, I, K, np.arange(8))
    assert np.array_equal(base["yq"], traded["yq"]) and np.array_equal(base["ys"], traded["ys"])
    ones = oracle.gemm_swiglu_rows_nvfp4(a, sa, w, ws, es, oracle.bf16_round_array(np.ones(8)), sfy, off, ids, I, K,
                                         np.arange(8))
    assert np.array_equal(base["yq"], ones["yq"]) and np.array_equal(base["ys"], ones["ys"])
