"""Pins for the oracle's grouped GEMM and fused SwiGLU (CPU only).

Fixes: hand-worked 1x1 cases (tests/golden), closed forms (constant and
one-hot rows), a per-group numpy float64 matmul over operands decoded by
torch (a library routine independent of the oracle's decoder and loops),
group-permutation equivariance, duplicate experts, zero-length groups,
and for SwiGLU the hand example, limits of silu and the fused == chained
identity the pages state for grouped_matmul_swiglu().
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


def torch_dec_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def torch_dec_e8m0(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e8m0fnu).double().numpy()


def dec_e2m1_table(packed):
    tab = np.array(GOLDEN["e2m1_values"]["codes_0_to_7"])
    tab = np.r_[tab, -tab]
    lo = tab[packed & 0xF]
    hi = tab[packed >> 4]
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


def rand_e4m3(rng, shape, lo=0x00, hi=0x7E):
    mag = rng.integers(lo, hi + 1, size=shape, dtype=np.int64)
    sign = rng.integers(0, 2, size=shape) * 0x80
    return (mag | sign).astype(np.uint8)


# ----------------------------------------------------------------------------- worked examples
def test_we4_rowwise_gemm_1x1():
    g = GOLDEN["WE4_rowwise_gemm_1x1"]
    K = g["K"]
    a = np.zeros((1, K), np.uint8)
    b = np.zeros((1, 1, K), np.uint8)
    a[0, :4] = [h(c) for c in g["a_codes_then_zeros"]]
    b[0, 0, :4] = [h(c) for c in g["b_codes_then_zeros"]]
    r = oracle.gemm_rows(0, a, np.array([g["a_scale"]], np.float32), b, np.array([[g["b_scale"]]], np.float32),
                         np.array([0, 1], np.uint32), np.array([0], np.int32), 1, K, [0])
    assert r["out"][0, 0] == h(g["out_bf16"])
    assert r["exact"][0, 0] == 0.375 and r["bound"][0, 0] == g["bound"]


def test_we5_mx_gemm_1x1():
    g = GOLDEN["WE5_mxfp8_gemm_1x1"]
    K = g["K"]
    a = np.full((1, K), h(g["a_code"]), np.uint8)
    b = np.full((1, 1, K), h(g["b_code"]), np.uint8)
    r = oracle.gemm_rows(1, a, np.full((1, 1), g["a_scale_code"], np.uint8), b,
                         np.full((1, 1, 1), g["b_scale_code"], np.uint8), np.array([0, 1], np.uint32),
                         np.array([0], np.int32), 1, K, [0])
    assert r["out"][0, 0] == h(g["out_bf16"])
    g = GOLDEN["WE5b_mxfp4_gemm_1x1"]
    a = np.full((1, K // 2), h(g["a_byte"]), np.uint8)
    b = np.full((1, 1, K // 2), h(g["b_byte"]), np.uint8)
    r = oracle.gemm_rows(2, a, np.full((1, 1), g["a_scale_code"], np.uint8), b,
                         np.full((1, 1, 1), g["b_scale_code"], np.uint8), np.array([0, 1], np.uint32),
                         np.array([0], np.int32), 1, K, [0])
    assert r["out"][0, 0] == h(g["out_bf16"])


# ----------------------------------------------------------------------------- closed forms
def test_constant_and_one_hot_rows():
    K, N = 96, 3
    a = np.zeros((2, K), np.uint8)
    a[0, :] = 0x40                       # 2.0 everywhere
    a[1, 37] = 0xB8                      # -1.0 only at k = 37
    b = np.zeros((1, N, K), np.uint8)
    b[0, 0, :] = 0x30                    # 0.5
    b[0, 1, :] = np.arange(K) % 0x7E
    b[0, 2, 37] = 0x7E                   # 448 at k = 37
    sa = np.array([0.25, 3.0], np.float32)
    sb = np.array([[2.0, 1.0, 0.5]], np.float32)
    r = oracle.gemm_rows(0, a, sa, b, sb, np.array([0, 2], np.uint32), np.array([0], np.int32), N, K, [0, 1])
    ex = r["exact"]
    assert ex[0, 0] == K * 2.0 * 0.5 * 0.25 * 2.0
    assert ex[0, 2] == 2.0 * 448 * 0.25 * 0.5
    assert ex[1, 0] == -0.5 * 3.0 * 2.0
    assert ex[1, 1] == -oracle.e4m3_value(37) * 3.0
    assert ex[1, 2] == -448 * 3.0 * 0.5


# ----------------------------------------------------------------------------- BLAS cross-check
def _ragged_case(rng, fmt, E=5, G=6, T=70, N=48, K=128):
    counts = rng.multinomial(T, np.ones(G) / G)
    counts[2] = 0                                   # an empty group
    off = np.r_[0, np.cumsum(counts)].astype(np.uint32)
    ids = rng.integers(0, E, size=G).astype(np.int32)
    ids[4] = ids[1]                                 # a duplicate expert
    T = int(off[-1])
    if fmt == 0:
        a = rand_e4m3(rng, (T, K))
        b = rand_e4m3(rng, (E, N, K))
        sa = (rng.random(T) * 0.01 + 1e-4).astype(np.float32)
        sb = (rng.random((E, N)) * 0.001 + 1e-5).astype(np.float32)
    elif fmt == 1:
        a = rand_e4m3(rng, (T, K))
        b = rand_e4m3(rng, (E, N, K))
        sa = rng.integers(110, 140, size=(T, K // 32)).astype(np.uint8)
        sb = rng.integers(110, 140, size=(E, N, K // 32)).astype(np.uint8)
    else:
        a = rng.integers(0, 256, size=(T, K // 2)).astype(np.uint8)
        b = rng.integers(0, 256, size=(E, N, K // 2)).astype(np.uint8)
        sa = rng.integers(110, 140, size=(T, K // 32)).astype(np.uint8)
        sb = rng.integers(110, 140, size=(E, N, K // 32)).astype(np.uint8)
    return dict(a=a, b=b, sa=sa, sb=sb, off=off, ids=ids, T=T, N=N, K=K, E=E, G=G)


def _blas_reference(fmt, c):
    """fp64 numpy matmul per group on torch-decoded (or table-decoded) operands."""
    T, N, K = c["T"], c["N"], c["K"]
    out = np.full((T, N), np.nan)
    for g in range(c["G"]):
        lo, hi = int(c["off"][g]), int(c["off"][g + 1])
        e = int(c["ids"][g])
        if fmt == 2:
            A = dec_e2m1_table(c["a"][lo:hi])
            B = dec_e2m1_table(c["b"][e])
        else:
            A = torch_dec_e4m3(c["a"][lo:hi])
            B = torch_dec_e4m3(c["b"][e])
        if fmt == 0:
            out[lo:hi] = (A @ B.T) * c["sa"][lo:hi, None].astype(np.float64) * c["sb"][e][None, :].astype(np.float64)
        else:
            SA = np.repeat(torch_dec_e8m0(c["sa"][lo:hi]), 32, axis=1)
            SB = np.repeat(torch_dec_e8m0(c["sb"][e]), 32, axis=1)
            out[lo:hi] = (A * SA) @ (B * SB).T
    return out


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_gemm_matches_numpy_float64_matmul(fmt):
    rng = np.random.default_rng(100 + fmt)
    c = _ragged_case(rng, fmt)
    ref = _blas_reference(fmt, c)
    r = oracle.gemm_rows(fmt, c["a"], c["sa"], c["b"], c["sb"], c["off"], c["ids"], c["N"], c["K"],
                         np.arange(c["T"]))
    assert np.all(r["group"] >= 0)
    np.testing.assert_allclose(r["exact"], ref, rtol=1e-12, atol=0)
    assert np.array_equal(r["out"], oracle.bf16_round_array(r["exact"]))


def test_gemm_group_permutation_equivariance_and_uncovered_rows():
    rng = np.random.default_rng(4)
    c = _ragged_case(rng, 0)
    base = oracle.gemm_rows(0, c["a"], c["sa"], c["b"], c["sb"], c["off"], c["ids"], c["N"], c["K"],
                            np.arange(c["T"]))
    # Reverse the group order by permuting the rows of A and the scale rows consistently.
    G = c["G"]
    perm_groups = list(range(G))[::-1]
    rows = np.concatenate([np.arange(c["off"][g], c["off"][g + 1]) for g in perm_groups]).astype(np.int64)
    counts = [int(c["off"][g + 1] - c["off"][g]) for g in perm_groups]
    off2 = np.r_[0, np.cumsum(counts)].astype(np.uint32)
    ids2 = c["ids"][perm_groups]
    r2 = oracle.gemm_rows(0, c["a"][rows], c["sa"][rows], c["b"], c["sb"], off2, ids2, c["N"], c["K"],
                          np.arange(c["T"]))
    assert np.array_equal(r2["out"], base["out"][rows])
    # a row beyond the last offset is not covered; an out-of-range expert id skips its group
    ids3 = c["ids"].copy()
    ids3[0] = c["E"]
    r3 = oracle.gemm_rows(0, c["a"], c["sa"], c["b"], c["sb"], c["off"], ids3, c["N"], c["K"],
                          np.arange(c["T"]))
    lo, hi = int(c["off"][0]), int(c["off"][1])
    assert np.all(r3["group"][lo:hi] == -1) and np.all(r3["group"][hi:] >= 0)


def test_gemm_rowwise_on_a_workload_slice_matches_blas():
    w = W.WORKLOADS[1]
    r = W.routing(w)
    x = W.activations(w, r)
    wt = W.weights(w)
    qa, sa = oracle.quantize(0, W.bf16_bits(x), r.row_offsets)
    qb, sb = oracle.quantize(0, W.bf16_bits(wt).reshape(w.E * w.N, w.K), np.array([0, w.E * w.N], np.uint32))
    qb = qb.reshape(w.E, w.N, w.K)
    sb = sb.reshape(w.E, w.N)
    c = dict(a=qa, b=qb, sa=sa, sb=sb, off=r.row_offsets, ids=r.expert_ids, T=r.total_rows, N=w.N, K=w.K,
             E=w.E, G=w.E)
    ref = _blas_reference(0, c)
    res = oracle.gemm_rows(0, qa, sa, qb, sb, r.row_offsets, r.expert_ids, w.N, w.K, np.arange(r.total_rows))
    np.testing.assert_allclose(res["exact"], ref, rtol=1e-12, atol=0)
    # quantization error stays small against the unquantized bf16 product
    xf = x.double().numpy()
    wf = wt.double().numpy()
    for g in range(w.E):
        lo, hi = int(r.row_offsets[g]), int(r.row_offsets[g + 1])
        full = xf[lo:hi] @ wf[g].T
        err = np.abs(res["exact"][lo:hi] - full).max() / np.abs(full).max()
        assert err < 0.1


# ----------------------------------------------------------------------------- SwiGLU
def test_we6_swiglu_requant():
    g = GOLDEN["WE6_swiglu_requant"]
    I = 32
    hrow = np.zeros((1, 2 * I), np.uint16)
    hrow[0, 0] = oracle.bf16_round(g["gate"])
    hrow[0, 1] = oracle.bf16_round(g["up"])
    yq, ys, y64 = oracle.silu_requant(hrow, np.array([0, 1], np.uint32), want_y64=True)
    assert oracle.bf16_round(y64[0, 0]) == h(g["y_bf16"])
    assert ys[0, 0] == g["scale_code"]
    assert (yq[0, 0] & 0xF) == h(g["nibble"]) and np.all(yq[0, 1:] == 0) and (yq[0, 0] >> 4) == 0


def test_silu_limits_and_gate_up_order():
    I = 32
    gate = np.array([0.0, 20.0, -20.0, 1.0, -1.0] + [0.0] * 27)
    up = np.array([5.0, 0.25, 3.0, -2.0, 2.0] + [0.0] * 27)
    hrow = np.zeros((1, 2 * I), np.uint16)
    hrow[0, 0::2] = oracle.bf16_round_array(gate)
    hrow[0, 1::2] = oracle.bf16_round_array(up)
    _, _, y = oracle.silu_requant(hrow, np.array([0, 1], np.uint32), want_y64=True)
    y = y[0]
    assert y[0] == 0.0
    assert abs(y[1] - 20.0 * 0.25) < 1e-7          # silu(z) -> z for large z
    assert abs(y[2]) < 1e-6 and y[2] < 0           # silu(z) -> 0- for very negative z
    assert abs(y[3] - (-2.0 / (1 + np.exp(-1.0)))) < 1e-15
    # swapping gate and up gives a different result (order is gate first)
    hswap = hrow.copy()
    hswap[0, 0::2], hswap[0, 1::2] = hrow[0, 1::2], hrow[0, 0::2]
    _, _, ys = oracle.silu_requant(hswap, np.array([0, 1], np.uint32), want_y64=True)
    assert not np.allclose(ys[0, :5], y[:5])


def test_fused_equals_chained_in_the_oracle():
    rng = np.random.default_rng(12)
    E, T, I, K = 3, 40, 64, 96
    off = np.array([0, 13, 13, 40], np.uint32)
    ids = np.array([2, 0, 1], np.int32)
    a = rng.integers(0, 256, size=(T, K // 2)).astype(np.uint8)
    w = rng.integers(0, 256, size=(E, 2 * I, K // 2)).astype(np.uint8)
    sa = rng.integers(120, 130, size=(T, K // 32)).astype(np.uint8)
    sw = rng.integers(120, 130, size=(E, 2 * I, K // 32)).astype(np.uint8)
    fused = oracle.gemm_swiglu_rows(2, a, sa, w, sw, off, ids, I, K, np.arange(T))
    gemm = oracle.gemm_rows(2, a, sa, w, sw, off, ids, 2 * I, K, np.arange(T))
    yq, ys = oracle.silu_requant(gemm["out"], off)
    assert np.array_equal(fused["yq"], yq) and np.array_equal(fused["ys"], ys)
    assert np.array_equal(fused["gu_exact"], gemm["exact"])
