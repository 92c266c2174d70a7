"""Pins for the oracle's padded / slot-strided MX scale layouts (CPU only).

The layout moves scale rows only, so the pins tie it to the (pinned) dense
quantize and GEMM: with scales_offsets = the group starts it is the dense
layout; with the expert-slot layout (offset = expert id * max_padded_M) every
group's scale rows equal the dense ones moved, the codes are unchanged, the
padding rows are never written, a row whose scale row falls past the tensor
is left untouched, and the GEMM is unchanged when its A scales come through
the same map.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def case(seed=1):
    w = W.WORKLOADS[5].scaled(tokens=40, E=6, masked=1, top_k=4, K=256, N=64, swiglu=False)
    r = W.routing(w)
    x = W.bf16_bits(W.activations(w, r))
    return w, r, x


@pytest.mark.parametrize("fmt", [oracle.MXFP8, oracle.MXFP4])
def test_identity_offsets_are_the_dense_layout(fmt):
    w, r, x = case()
    T = x.shape[0]
    qd, sd = oracle.quantize(fmt, x, r.row_offsets)
    qp, sp = oracle.quantize_padded(fmt, x, r.row_offsets, r.row_offsets[:-1], T)
    assert np.array_equal(qd, qp) and np.array_equal(sd, sp)


@pytest.mark.parametrize("fmt", [oracle.MXFP8, oracle.MXFP4])
def test_slot_layout_moves_scale_rows(fmt):
    w, r, x = case()
    K = x.shape[1]
    counts = np.diff(r.row_offsets.astype(np.int64))
    mpad = int(-(-counts.max() // 128) * 128)          # slot height: max rows rounded up to 128
    soff = (r.expert_ids.astype(np.int64) * mpad).astype(np.uint32)
    S = int(w.E * mpad)
    qd, sd = oracle.quantize(fmt, x, r.row_offsets)
    qp, sp = oracle.quantize_padded(fmt, x, r.row_offsets, soff, S, scales=np.full((S, K // 32), 0x5A, np.uint8))
    assert np.array_equal(qd, qp)
    written = np.zeros(S, bool)
    for g in range(len(r.expert_ids)):
        lo, hi = int(r.row_offsets[g]), int(r.row_offsets[g + 1])
        assert np.array_equal(sp[soff[g]:soff[g] + hi - lo], sd[lo:hi])
        written[soff[g]:soff[g] + hi - lo] = True
    assert np.all(sp[~written] == 0x5A)


def test_rows_past_the_scale_tensor_are_untouched():
    w, r, x = case()
    T, K = x.shape
    soff = r.row_offsets[:-1].copy()
    S = T - 5                                          # the last 5 routed rows have no scale row
    q0 = np.full((T, K), 0xA5, np.uint8)
    qp, sp = oracle.quantize_padded(oracle.MXFP8, x, r.row_offsets, soff, S, q=q0.copy())
    qd, sd = oracle.quantize(oracle.MXFP8, x, r.row_offsets)
    assert np.array_equal(qp[:S], qd[:S]) and np.all(qp[S:] == 0xA5)


@pytest.mark.parametrize("fmt", [oracle.MXFP8, oracle.MXFP4])
def test_gemm_with_moved_scales_is_unchanged(fmt):
    w, r, x = case()
    T, K = x.shape
    a, sd = oracle.quantize(fmt, x, r.row_offsets)
    rng = np.random.default_rng(5)
    wt = oracle.bf16_round_array(rng.normal(0, 0.02, size=(w.E * w.N, K)))
    b, sb = oracle.quantize(fmt, wt, np.array([0, w.E * w.N], np.uint32))
    b = b.reshape(w.E, w.N, -1)
    sb = sb.reshape(w.E, w.N, -1)
    counts = np.diff(r.row_offsets.astype(np.int64))
    mpad = int(-(-counts.max() // 64) * 64)
    soff = (r.expert_ids.astype(np.int64) * mpad).astype(np.uint32)
    _, sp = oracle.quantize_padded(fmt, x, r.row_offsets, soff, w.E * mpad)
    rows = np.arange(T)
    dense = oracle.gemm_rows(fmt, a, sd, b, sb, r.row_offsets, r.expert_ids, w.N, K, rows)
    padded = oracle.gemm_rows_padded(fmt, a, sp, soff, b, sb, r.row_offsets, r.expert_ids, w.N, K, rows)
    assert np.array_equal(dense["group"], padded["group"])
    cov = dense["group"] >= 0
    assert np.array_equal(dense["exact"][cov], padded["exact"][cov])


def nv_case():
    w, r, x = case()
    sf = np.linspace(50.0, 2688.0, w.E).astype(np.float32)
    return w, r, x, sf


def test_nvfp4_identity_offsets_are_the_dense_layout():
    w, r, x, sf = nv_case()
    T = x.shape[0]
    qd, sd = oracle.quantize_nvfp4(x, r.row_offsets, r.expert_ids, sf)
    qp, sp = oracle.quantize_nvfp4_padded(x, r.row_offsets, r.expert_ids, sf, r.row_offsets[:-1], T)
    cov = np.zeros(T, bool)
    for g in range(len(r.expert_ids)):
        cov[r.row_offsets[g]:r.row_offsets[g + 1]] = True
    assert np.array_equal(qd[cov], qp[cov]) and np.array_equal(sd[cov], sp[cov])


def test_nvfp4_slot_layout_moves_scale_rows_and_cuts_at_the_end():
    """NVFP4 scales (16-element blocks) in the expert-slot layout: codes as the
    dense quantize, each group's scale rows moved to its slot, padding rows
    never written; with the tensor cut inside a slot, the rows past the cut
    are left untouched, codes included."""
    w, r, x, sf = nv_case()
    T, K = x.shape
    counts = np.diff(r.row_offsets.astype(np.int64))
    mpad = int(-(-counts.max() // 64) * 64)
    soff = (r.expert_ids.astype(np.int64) * mpad).astype(np.uint32)
    S = int(w.E * mpad)
    qd, sd = oracle.quantize_nvfp4(x, r.row_offsets, r.expert_ids, sf)
    qp, sp = oracle.quantize_nvfp4_padded(x, r.row_offsets, r.expert_ids, sf, soff, S,
                                          scales=np.full((S, K // 16), 0x5A, np.uint8))
    written = np.zeros(S, bool)
    for g in range(len(r.expert_ids)):
        lo, hi = int(r.row_offsets[g]), int(r.row_offsets[g + 1])
        assert np.array_equal(qp[lo:hi], qd[lo:hi])
        assert np.array_equal(sp[soff[g]:soff[g] + hi - lo], sd[lo:hi])
        written[soff[g]:soff[g] + hi - lo] = True
    assert np.all(sp[~written] == 0x5A)
    g = int(np.argmax(counts))
    cut = int(soff[g]) + int(counts[g]) // 2
    q0 = np.full((T, K // 2), 0xA5, np.uint8)
    qc, sc = oracle.quantize_nvfp4_padded(x, r.row_offsets, r.expert_ids, sf, soff, cut, q0.copy(),
                                          np.full((cut, K // 16), 0x5A, np.uint8))
    for gg in range(len(r.expert_ids)):
        lo, hi = int(r.row_offsets[gg]), int(r.row_offsets[gg + 1])
        for t in range(lo, hi):
            if int(soff[gg]) + t - lo < cut:
                assert np.array_equal(qc[t], qd[t]) and np.array_equal(sc[int(soff[gg]) + t - lo], sd[t])
            else:
                assert np.all(qc[t] == 0xA5)
