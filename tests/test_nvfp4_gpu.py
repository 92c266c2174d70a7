"""GPU parity for the NVFP4 path: the grouped quantize must match the CPU
oracle bit for bit (codes and E4M3 block scales) and leave rows of skipped
or uncovered groups untouched."""
import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import oracle
import workloads as W
from common import Guarded, bits, offsets_gpu, sentinel_like, to_gpu

pytestmark = pytest.mark.gpu


def tensor_scales(x_bits, off, ids, E, seed):
    """Calibration-like per-expert tensor scales: 448 * 6 / (largest |x| of the
    expert's rows), times a seeded factor in [0.5, 2] so that saturating and
    non-power-of-two block scales occur.  (An input choice, not the method.)"""
    xv = oracle.bf16_value_array(x_bits)
    amax = np.ones(E)
    for g in range(len(ids)):
        lo, hi = int(off[g]), int(off[g + 1])
        if 0 <= ids[g] < E and hi > lo:
            amax[ids[g]] = max(np.abs(xv[lo:hi]).max(), 1e-30)
    f = np.random.default_rng(seed).uniform(0.5, 2.0, size=E)
    return (448.0 * 6.0 / amax * f).astype(np.float32)


def run_both(x_bits, off, ids, sf):
    T, K = x_bits.shape
    q_ref, s_ref = oracle.quantize_nvfp4(x_bits, off, ids, sf, sentinel_like((T, K // 2)),
                                         sentinel_like((T, K // 16), value=0x5A))
    x = to_gpu(x_bits.view(np.int16)).view(torch.bfloat16)
    q = to_gpu(sentinel_like((T, K // 2)))
    s = to_gpu(sentinel_like((T, K // 16), value=0x5A))
    mxg.mx_grouped_quantize_nvfp4(x, q, s, to_gpu(sf), offsets_gpu(off), to_gpu(ids.astype(np.int32)))
    torch.cuda.synchronize()
    return (q.cpu().numpy(), s.cpu().numpy()), (q_ref, s_ref)


def assert_same(gpu, ref, label):
    (q, s), (qr, sr) = gpu, ref
    bad = np.argwhere(q != qr)
    assert bad.size == 0, f"{label}: {len(bad)} code bytes differ, first at {bad[0]}: gpu {q[tuple(bad[0])]:#x} oracle {qr[tuple(bad[0])]:#x}"
    bad = np.argwhere(s != sr)
    assert bad.size == 0, f"{label}: {len(bad)} scale bytes differ, first at {bad[0]}: gpu {s[tuple(bad[0])]:#x} oracle {sr[tuple(bad[0])]:#x}"


@pytest.mark.parametrize("K", [16, 48, 512, 1040, 7168, 8704])
def test_quantize_nvfp4_matches_oracle(K):
    w = W.WORKLOADS[5].scaled(tokens=40, E=8, masked=1, top_k=4, K=K)
    r = W.routing(w)
    x = bits(W.activations(w, r))
    E = w.E
    sf = tensor_scales(x, r.row_offsets, r.expert_ids, E, seed=K)
    gpu, ref = run_both(x, r.row_offsets, r.expert_ids, sf)
    assert_same(gpu, ref, f"K={K}")


def test_quantize_nvfp4_special_values():
    """Zero rows, tiny blocks that underflow, blocks that saturate the E4M3 scale."""
    T, K = 6, 64
    xv = np.zeros((T, K))
    xv[1, :16] = 2.0 ** -14                               # underflow with sf = 1
    xv[2, :] = np.linspace(-600, 600, K)                  # saturating block scales with sf = 6
    xv[3, ::2] = -0.0
    xv[4, :] = np.random.default_rng(1).normal(size=K) * 1e-3
    xv[5, 16:32] = 6.0
    x = oracle.bf16_round_array(xv)
    off = np.array([0, 2, 3, 6], np.uint32)
    ids = np.array([0, 1, 2], np.int32)
    sf = np.array([1.0, 6.0, 1000.0], np.float32)
    gpu, ref = run_both(x, off, ids, sf)
    assert_same(gpu, ref, "special")


def test_quantize_nvfp4_skips_bad_expert_ids_and_uncovered_rows():
    T, K = 48, 64
    x = bits(torch.randn(T, K).to(torch.bfloat16))
    off = np.array([0, 10, 10, 30, 40], np.uint32)        # rows 40..47 uncovered, group 1 empty
    ids = np.array([1, 0, 7, 2], np.int32)                # expert 7 is out of range (E = 3)
    sf = np.array([100.0, 50.0, 25.0], np.float32)
    gpu, ref = run_both(x, off, ids, sf)
    assert_same(gpu, ref, "skips")
    # rows of the skipped group (10..29) and the uncovered rows (40..47) keep their sentinels
    for rows in (slice(10, 30), slice(40, 48)):
        assert np.all(gpu[0][rows] == 0xA5) and np.all(gpu[1][rows] == 0x5A)


def test_quantize_nvfp4_full_size_sampled_rows():
    """The mxfp4_swiglu routing and shape (32,768 x 7168) in NVFP4; sampled rows
    checked against the oracle run on those rows (each with its group's scale)."""
    w = W.WORKLOADS[5]
    r = W.routing(w)
    x_gpu = W.activations(w, r, device="cuda")
    T, K = x_gpu.shape
    E = w.E
    xb = bits(x_gpu.cpu())
    sf = tensor_scales(xb, r.row_offsets, r.expert_ids, E, seed=5)
    q, s = mxg.quantize_nvfp4(x_gpu, offsets_gpu(r.row_offsets), to_gpu(r.expert_ids.astype(np.int32)), to_gpu(sf))
    torch.cuda.synchronize()
    rng = np.random.default_rng(55)
    rows = []
    for g in range(len(r.expert_ids)):
        lo, hi = int(r.row_offsets[g]), int(r.row_offsets[g + 1])
        if hi > lo:
            rows += [lo, hi - 1]
    rows = np.unique(np.array(rows + list(rng.integers(0, T, 64))))
    grp = np.searchsorted(r.row_offsets[1:], rows, side="right")
    off1 = np.arange(rows.size + 1, dtype=np.uint32)
    qr, sr = oracle.quantize_nvfp4(xb[rows], off1, r.expert_ids[grp].astype(np.int32), sf)
    assert_same((q.cpu().numpy()[rows], s.cpu().numpy()[rows]), (qr, sr), "full size")


# ----------------------------------------------------------------------------- grouped GEMM
from common import check_gemm_rows  # noqa: E402

SENT_BF16 = 0x7FA5  # a NaN pattern no result can produce


def nv_gemm_inputs(w, seed, quantized=True):
    """NVFP4 operands for workload w.  quantized: codes and scales from the
    oracle's quantize of the seeded activations / weights (tensor scales as in
    the quantize tests); otherwise seeded random codes and E4M3 scales."""
    r = W.routing(w)
    T, E, N, K = r.total_rows, w.E, w.N, w.K
    rng = np.random.default_rng(seed)
    if quantized:
        x = bits(W.activations(w, r))
        sfa = tensor_scales(x, r.row_offsets, r.expert_ids, E, seed=seed)
        a, sa = oracle.quantize_nvfp4(x, r.row_offsets, r.expert_ids, sfa)
        wt = bits(W.weights(w)).reshape(E * N, K)
        off_w = np.arange(0, (E + 1) * N, N, dtype=np.uint32)
        ids_w = np.arange(E, dtype=np.int32)
        sfw = tensor_scales(wt, off_w, ids_w, E, seed=seed + 1)
        b, sb = oracle.quantize_nvfp4(wt, off_w, ids_w, sfw)
        b, sb = b.reshape(E, N, K // 2), sb.reshape(E, N, K // 16)
        es = (1.0 / (sfa.astype(np.float64) * sfw)).astype(np.float32)
    else:
        a = rng.integers(0, 256, size=(T, K // 2), dtype=np.uint8)
        sa = rng.integers(0x28, 0x48, size=(T, K // 16), dtype=np.uint8)
        b = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        sb = rng.integers(0x28, 0x48, size=(E, N, K // 16), dtype=np.uint8)
        es = rng.uniform(0.25, 4.0, size=E).astype(np.float32)
    return r, a, sa, b, sb, es


def run_nv_gemm(r, a, sa, b, sb, es, hint=0):
    T, N = a.shape[0], b.shape[1]
    g = Guarded(np.full((T, N), SENT_BF16, np.uint16))
    mxg.mx_grouped_matmul_nvfp4(to_gpu(a), to_gpu(sa), to_gpu(b), to_gpu(sb), to_gpu(es), g.view(torch.bfloat16),
                                offsets_gpu(r.row_offsets), to_gpu(r.expert_ids.astype(np.int32)), hint)
    torch.cuda.synchronize()
    g.check("NVFP4 c")
    return g.numpy()


NV_SMALL = {
    # several M and N tiles, ragged M tails, a partial N tile, an empty (masked) expert
    "k512": W.WORKLOADS[5].scaled(tokens=96, E=8, masked=1, top_k=4, N=288, K=512, swiglu=False),
    "k1024": W.WORKLOADS[5].scaled(tokens=80, E=6, masked=1, top_k=4, N=320, K=1024, swiglu=False),
    "k2048_tall": W.WORKLOADS[5].scaled(tokens=512, E=4, masked=0, top_k=2, N=256, K=2048, swiglu=False),
}


@pytest.mark.parametrize("name", list(NV_SMALL))
def test_nvfp4_gemm_matches_oracle_all_rows(name):
    w = NV_SMALL[name]
    r, a, sa, b, sb, es = nv_gemm_inputs(w, seed=21)
    c = run_nv_gemm(r, a, sa, b, sb, es)
    rows = np.arange(a.shape[0])
    ref = oracle.gemm_rows_nvfp4(a, sa, b, sb, es, r.row_offsets, r.expert_ids, w.N, w.K, rows)
    cov = ref["group"] >= 0
    assert np.all(c[~cov] == SENT_BF16), "uncovered rows were written"
    worst, exact = check_gemm_rows(c[cov], {k: v[cov] for k, v in ref.items() if k != "group"}, name)
    print(f"{name}: max |err|/tol = {worst:.3g}, bf16-exact = {exact:.4f}")
    assert exact > 0.9


def test_nvfp4_gemm_random_codes_and_bad_expert_ids():
    """Random codes and block scales (every e2m1 code, a wide E4M3 range); a
    group with an out-of-range expert id leaves its rows untouched."""
    w = W.WORKLOADS[5].scaled(tokens=64, E=5, masked=0, top_k=4, N=256, K=1024, swiglu=False)
    r, a, sa, b, sb, es = nv_gemm_inputs(w, seed=4, quantized=False)
    r.expert_ids = r.expert_ids.copy()
    r.expert_ids[1] = 9
    c = run_nv_gemm(r, a, sa, b, sb, es)
    ref = oracle.gemm_rows_nvfp4(a, sa, b, sb, es, r.row_offsets, r.expert_ids, w.N, w.K, np.arange(a.shape[0]))
    cov = ref["group"] >= 0
    assert (~cov).any() and np.all(c[~cov] == SENT_BF16)
    check_gemm_rows(c[cov], {k: v[cov] for k, v in ref.items() if k != "group"}, "random codes")


# Sparse and malformed routings (as in the MX / FP8 ragged suite): groups
# with an id outside [0, E) or inverted offsets are skipped, offsets past the
# end are clamped to T, rows no valid group covers keep the sentinel.
NV_GROUPINGS = {
    "empty_groups": ([0, 0, 50, 50, 50, 130, 130], [0, 1, 2, 3, 1, 0]),
    "subset_with_gaps": ([5, 40, 40, 90], [1, 1, 2]),
    "out_of_range_ids": ([0, 40, 80, 130], [4, -1, 1]),
    "inverted_and_past_end": ([60, 20, 100, 500], [0, 1, 2]),
}


@pytest.mark.parametrize("K", [512, 1024])
@pytest.mark.parametrize("name", list(NV_GROUPINGS))
def test_nvfp4_gemm_sparse_and_malformed_routing(name, K):
    rng = np.random.default_rng(len(name) * 13 + K)
    T, E, N = 130, 4, 288
    a = rng.integers(0, 256, size=(T, K // 2), dtype=np.uint8)
    sa = rng.integers(0x28, 0x48, size=(T, K // 16), dtype=np.uint8)
    b = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    sb = rng.integers(0x28, 0x48, size=(E, N, K // 16), dtype=np.uint8)
    es = rng.uniform(0.25, 4.0, size=E).astype(np.float32)
    off = np.array(NV_GROUPINGS[name][0], np.uint32)
    ids = np.array(NV_GROUPINGS[name][1], np.int32)
    g = Guarded(np.full((T, N), SENT_BF16, np.uint16))
    mxg.mx_grouped_matmul_nvfp4(to_gpu(a), to_gpu(sa), to_gpu(b), to_gpu(sb), to_gpu(es), g.view(torch.bfloat16),
                                offsets_gpu(off), to_gpu(ids))
    torch.cuda.synchronize()
    g.check("NVFP4 c")
    c = g.numpy()
    ref = oracle.gemm_rows_nvfp4(a, sa, b, sb, es, off, ids, N, K, np.arange(T))
    cov = ref["group"] >= 0
    assert np.all(c[~cov] == SENT_BF16), "a row no valid group covers was written"
    if cov.any():
        check_gemm_rows(c[cov], {k: v[cov] for k, v in ref.items() if k != "group"}, name)


def test_nvfp4_gemm_full_size_sampled_rows():
    """The mxfp4_swiglu routing at full size (32,768 routed rows, 128 experts,
    K = 7168) as a plain NVFP4 GEMM with N = 4096; seeded random operands,
    sampled rows (first / last of every group and random ones)."""
    w = W.WORKLOADS[5].scaled(swiglu=False)
    r, a, sa, b, sb, es = nv_gemm_inputs(w, seed=8, quantized=False)
    c = run_nv_gemm(r, a, sa, b, sb, es, hint=int(r.counts.max()))
    rng = np.random.default_rng(88)
    rows = []
    for g in range(len(r.expert_ids)):
        lo, hi = int(r.row_offsets[g]), int(r.row_offsets[g + 1])
        if hi > lo:
            rows += [lo, hi - 1]
    rows = np.unique(np.array(rows + list(rng.integers(0, a.shape[0], 32))))
    ref = oracle.gemm_rows_nvfp4(a, sa, b, sb, es, r.row_offsets, r.expert_ids, w.N, w.K, rows)
    worst, exact = check_gemm_rows(c[rows], ref, "full size")
    print(f"full size: {rows.size} rows, max |err|/tol = {worst:.3g}, bf16-exact = {exact:.4f}")


# ----------------------------------------------------------------------------- SwiGLU + NVFP4 requant
from common import _silu_range, gemm_tolerance  # noqa: E402

E2M1_TAB = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)


def fragile_mask(y64, rel=2.0**-20):
    return oracle.bf16_round_array(y64 * (1 - rel)) != oracle.bf16_round_array(y64 * (1 + rel))


def nibbles(q):
    return np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1)


def check_requant_exact(yq, ys, yq_ref, ys_ref, y64):
    """Bit-exact except in blocks holding an element whose fp64 y lies within
    2^-20 (relative) of a bf16 rounding boundary (the GPU evaluates silu in fp32)."""
    n, I = y64.shape
    frag_blk = fragile_mask(y64).reshape(n, I // 16, 16).any(axis=2)
    assert np.array_equal(ys[~frag_blk], ys_ref[~frag_blk]), "block scales differ in non-fragile blocks"
    strict = np.repeat(~frag_blk & (ys == ys_ref), 16, axis=1)
    assert np.array_equal(nibbles(yq)[strict], nibbles(yq_ref)[strict]), "codes differ in non-fragile blocks"
    return float(frag_blk.mean())


def check_nv_swiglu_interval(yq, ys, gu_exact, gu_bound, sf_rows):
    """The fused result must be reachable from SOME gate/up pair inside the GEMM
    tolerance: its E4M3 block scale must come from an amax in the block's
    interval, and each code must be the rounding of some y in the element's
    interval under that scale (the encode steps are monotone)."""
    tol = gemm_tolerance(gu_exact, gu_bound)
    lo = oracle.bf16_value_array(oracle.bf16_round_array(gu_exact - tol))
    hi = oracle.bf16_value_array(oracle.bf16_round_array(gu_exact + tol))
    s_lo, s_hi = _silu_range(lo[:, 0::2], hi[:, 0::2])
    u_lo, u_hi = lo[:, 1::2], hi[:, 1::2]
    corners = np.stack([s_lo * u_lo, s_lo * u_hi, s_hi * u_lo, s_hi * u_hi])
    c_min, c_max = corners.min(axis=0), corners.max(axis=0)
    c_min = c_min - np.abs(c_min) * 2.0**-20
    c_max = c_max + np.abs(c_max) * 2.0**-20
    y_lo = oracle.bf16_value_array(oracle.bf16_round_array(c_min))
    y_hi = oracle.bf16_value_array(oracle.bf16_round_array(c_max))
    n, I = y_lo.shape
    amag_hi = np.maximum(np.abs(y_lo), np.abs(y_hi)).reshape(n, I // 16, 16).max(axis=2)
    amag_lo = np.where((y_lo <= 0) & (y_hi >= 0), 0.0,
                       np.minimum(np.abs(y_lo), np.abs(y_hi))).reshape(n, I // 16, 16).max(axis=2)
    sf = np.asarray(sf_rows, np.float32)[:, None]

    def scale_code(amag):
        u = (amag.astype(np.float32) / np.float32(6.0)) * sf
        return oracle.e4m3_encode_array(np.minimum(u, np.float32(448.0)).astype(np.float64)).astype(np.int64)

    c_lo_s, c_hi_s = scale_code(amag_lo), scale_code(amag_hi)
    sc = ys.astype(np.int64)
    bad = (sc < c_lo_s) | (sc > c_hi_s)
    if bad.any():
        i, b = np.argwhere(bad)[0]
        raise AssertionError(f"scale outside interval at row {i} block {b}: gpu {sc[i, b]:#x} "
                             f"allowed [{c_lo_s[i, b]:#x}, {c_hi_s[i, b]:#x}]")
    sval = oracle.e4m3_value_array(ys.astype(np.uint8)).astype(np.float32)
    r = np.where(sval == 0, np.float32(0), sf / np.where(sval == 0, np.float32(1), sval)).astype(np.float32)
    rr = np.repeat(r, 16, axis=1)
    e_lo = E2M1_TAB[oracle.e2m1_encode_array((y_lo.astype(np.float32) * rr).astype(np.float64))]
    e_hi = E2M1_TAB[oracle.e2m1_encode_array((y_hi.astype(np.float32) * rr).astype(np.float64))]
    val = E2M1_TAB[nibbles(yq)]
    bad = (val < np.minimum(e_lo, e_hi)) | (val > np.maximum(e_lo, e_hi))
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"code outside interval at row {i} output {j}: gpu {val[i, j]} "
                             f"allowed [{e_lo[i, j]}, {e_hi[i, j]}]")


@pytest.mark.parametrize("I,T", [(16, 17), (1024, 96), (80, 300)])
def test_silu_quantize_nvfp4_matches_oracle(I, T):
    rng = np.random.default_rng(I + T)
    vals = rng.standard_normal((T, 2 * I)) * np.exp(rng.uniform(-6, 4, (T, 1)))
    vals[0, :8] = [0.0, 5.0, -0.0, 3.0, 1.0, 2.0, -20.0, 4.0]
    h = oracle.bf16_round_array(vals)
    # groups: [0, 3) expert 1, an empty one, [3, T-8) with an out-of-range id (skipped),
    # [T-8, T-4) expert 0; the last 4 rows are uncovered
    off = np.array([0, 3, 3, T - 8, T - 4], np.uint32)
    ids = np.array([1, 0, 5, 0], np.int32)
    sfy = np.array([0.5, 300.0], np.float32)
    yq_ref, ys_ref, y64 = oracle.silu_requant_nvfp4(h, off, ids, sfy, np.full((T, I // 2), 0xA5, np.uint8),
                                                    np.full((T, I // 16), 0x5A, np.uint8), want_y64=True)
    hg = to_gpu(h.view(np.int16)).view(torch.bfloat16)
    yq = torch.full((T, I // 2), 0xA5, dtype=torch.uint8, device="cuda")
    ys = torch.full((T, I // 16), 0x5A, dtype=torch.uint8, device="cuda")
    mxg.mx_silu_quantize_nvfp4(hg, yq, ys, to_gpu(sfy), offsets_gpu(off), to_gpu(ids))
    yq, ys = yq.cpu().numpy(), ys.cpu().numpy()
    cov = np.zeros(T, bool)
    cov[0:3] = True
    cov[T - 8:T - 4] = True
    assert np.all(yq[~cov] == 0xA5) and np.all(ys[~cov] == 0x5A)
    frac = check_requant_exact(yq[cov], ys[cov], yq_ref[cov], ys_ref[cov], y64[cov])
    print(f"fragile block fraction {frac:.2e}")


def nv_swiglu_inputs(w, seed, quantized=True):
    r, a, sa, b, sb, es = nv_gemm_inputs(w, seed, quantized)
    sfy = np.random.default_rng(seed + 7).uniform(0.5, 500.0, size=w.E).astype(np.float32)
    return r, a, sa, b, sb, es, sfy


def run_nv_fused(r, a, sa, b, sb, es, sfy, rs=None, hint=0):
    T, I = a.shape[0], b.shape[1] // 2
    gq = Guarded(np.full((T, I // 2), 0xA5, np.uint8))
    gs = Guarded(np.full((T, I // 16), 0x5A, np.uint8))
    rs_g = None if rs is None else to_gpu(rs.view(np.int16)).view(torch.bfloat16)
    mxg.mx_grouped_matmul_swiglu_nvfp4(to_gpu(a), to_gpu(sa), to_gpu(b), to_gpu(sb), to_gpu(es), to_gpu(sfy),
                                       gq.view(), gs.view(), offsets_gpu(r.row_offsets),
                                       to_gpu(r.expert_ids.astype(np.int32)), rs_g, hint)
    torch.cuda.synchronize()
    gq.check("NVFP4 fused codes")
    gs.check("NVFP4 fused scales")
    return gq.numpy(), gs.numpy()


def run_nv_chained(r, a, sa, b, sb, es, sfy):
    T, N = a.shape[0], b.shape[1]
    c = torch.zeros((T, N), dtype=torch.bfloat16, device="cuda")
    off, ids = offsets_gpu(r.row_offsets), to_gpu(r.expert_ids.astype(np.int32))
    mxg.mx_grouped_matmul_nvfp4(to_gpu(a), to_gpu(sa), to_gpu(b), to_gpu(sb), to_gpu(es), c, off, ids)
    yq = torch.full((T, N // 4), 0xA5, dtype=torch.uint8, device="cuda")
    ys = torch.full((T, N // 32), 0x5A, dtype=torch.uint8, device="cuda")
    mxg.mx_silu_quantize_nvfp4(c, yq, ys, to_gpu(sfy), off, ids)
    torch.cuda.synchronize()
    return yq.cpu().numpy(), ys.cpu().numpy()


NV_FUSED = {
    "k512": W.WORKLOADS[5].scaled(tokens=96, E=8, masked=1, top_k=4, N=320, K=512),
    "k1024_tall": W.WORKLOADS[5].scaled(tokens=512, E=4, masked=0, top_k=2, N=256, K=1024),
}


@pytest.mark.parametrize("name", list(NV_FUSED))
def test_nvfp4_fused_equals_chained_and_oracle(name):
    w = NV_FUSED[name]
    r, a, sa, b, sb, es, sfy = nv_swiglu_inputs(w, seed=31)
    yq, ys = run_nv_fused(r, a, sa, b, sb, es, sfy)
    yq2, ys2 = run_nv_chained(r, a, sa, b, sb, es, sfy)
    assert np.array_equal(yq, yq2) and np.array_equal(ys, ys2), "fused and chained NVFP4 paths differ"
    rows = np.arange(a.shape[0])
    ref = oracle.gemm_swiglu_rows_nvfp4(a, sa, b, sb, es, None, sfy, r.row_offsets, r.expert_ids, w.N // 2, w.K, rows)
    cov = ref["group"] >= 0
    assert np.all(yq[~cov] == 0xA5) and np.all(ys[~cov] == 0x5A)
    sf_rows = sfy[r.expert_ids[ref["group"][cov]]]
    check_nv_swiglu_interval(yq[cov], ys[cov], ref["gu_exact"][cov], ref["gu_bound"][cov], sf_rows)
    same = np.mean(ys[cov] == ref["ys"][cov])
    print(f"{name}: scale bytes equal to the oracle's {same:.4f}")
    assert same > 0.95


def test_nvfp4_fused_with_row_scales_vs_oracle():
    w = NV_FUSED["k512"]
    r, a, sa, b, sb, es, sfy = nv_swiglu_inputs(w, seed=37)
    rs = oracle.bf16_round_array(np.random.default_rng(3).uniform(0.25, 4.0, a.shape[0]))
    yq, ys = run_nv_fused(r, a, sa, b, sb, es, sfy, rs=rs)
    rows = np.arange(a.shape[0])
    ref = oracle.gemm_swiglu_rows_nvfp4(a, sa, b, sb, es, rs, sfy, r.row_offsets, r.expert_ids, w.N // 2, w.K, rows)
    cov = ref["group"] >= 0
    check_nv_swiglu_interval(yq[cov], ys[cov], ref["gu_exact"][cov], ref["gu_bound"][cov],
                             sfy[r.expert_ids[ref["group"][cov]]])
    assert np.mean(ys[cov] == ref["ys"][cov]) > 0.95


def test_nvfp4_fused_full_size_sampled_rows():
    """The mxfp4_swiglu routing and shape (32,768 rows, I = 2048, K = 7168) in
    NVFP4, seeded random operands: fused == chained on every row, and sampled
    rows inside the oracle's intervals."""
    w = W.WORKLOADS[5]
    r, a, sa, b, sb, es, sfy = nv_swiglu_inputs(w, seed=41, quantized=False)
    yq, ys = run_nv_fused(r, a, sa, b, sb, es, sfy, hint=int(r.counts.max()))
    yq2, ys2 = run_nv_chained(r, a, sa, b, sb, es, sfy)
    assert np.array_equal(yq, yq2) and np.array_equal(ys, ys2), "fused and chained NVFP4 paths differ"
    rng = np.random.default_rng(42)
    rows = []
    for g in range(len(r.expert_ids)):
        lo, hi = int(r.row_offsets[g]), int(r.row_offsets[g + 1])
        if hi > lo:
            rows += [lo, hi - 1]
    rows = np.unique(np.array(rows + list(rng.integers(0, a.shape[0], 16))))
    ref = oracle.gemm_swiglu_rows_nvfp4(a, sa, b, sb, es, None, sfy, r.row_offsets, r.expert_ids, w.N // 2, w.K, rows)
    check_nv_swiglu_interval(yq[rows], ys[rows], ref["gu_exact"], ref["gu_bound"], sfy[r.expert_ids[ref["group"]]])


# ---------------------------------------------------------------- padded / slot-strided NVFP4 scales
def nv_slot_offsets(r, round_to=64):
    counts = np.diff(r.row_offsets.astype(np.int64))
    mpad = int(max(1, -(-counts.max() // round_to)) * round_to)
    return (r.expert_ids.astype(np.int64) * mpad).astype(np.uint32), mpad


@pytest.mark.parametrize("K", [512, 7168])
def test_quantize_nvfp4_padded_matches_oracle(K):
    """NVFP4 scales in the expert-slot layout, bit for bit with the oracle; the
    padding rows and, with the tensor cut inside a slot, the rows past the cut
    (codes included) are left untouched."""
    w = W.WORKLOADS[5].scaled(tokens=48, E=6, masked=1, top_k=4, K=K)
    r = W.routing(w)
    x = bits(W.activations(w, r))
    T = x.shape[0]
    sf = tensor_scales(x, r.row_offsets, r.expert_ids, w.E, seed=K)
    soff, mpad = nv_slot_offsets(r)
    counts = np.diff(r.row_offsets.astype(np.int64))
    g = int(np.argmax(counts))
    for S in (w.E * mpad, int(soff[g]) + int(counts[g]) // 2 + 3):
        q_ref, s_ref = oracle.quantize_nvfp4_padded(x, r.row_offsets, r.expert_ids, sf, soff, S,
                                                    sentinel_like((T, K // 2)), sentinel_like((S, K // 16), value=0x5A))
        q = Guarded(sentinel_like((T, K // 2)))
        s = Guarded(sentinel_like((S, K // 16), value=0x5A))
        mxg.mx_grouped_quantize_nvfp4_padded(to_gpu(x.view(np.int16)).view(torch.bfloat16), q.view(), s.view(),
                                             to_gpu(sf), to_gpu(soff), offsets_gpu(r.row_offsets),
                                             to_gpu(r.expert_ids.astype(np.int32)))
        torch.cuda.synchronize()
        q.check("codes")
        s.check("scales")
        assert_same((q.numpy(), s.numpy()), (q_ref, s_ref), f"NVFP4 padded K={K} S={S}")


@pytest.mark.parametrize("hint", [0, 1 << 20])
def test_nvfp4_gemm_padded_equals_dense_and_oracle(hint):
    """The NVFP4 GEMM reading A's scales through the slot layout equals the
    dense-layout GEMM bit for bit; with the scale tensor cut inside a group,
    rows without scale rows are left untouched and the rest match the oracle."""
    w = NV_SMALL["k1024"]
    r, a, sa, b, sb, es = nv_gemm_inputs(w, seed=23)
    T, K, N = a.shape[0], w.K, w.N
    soff, mpad = nv_slot_offsets(r)
    S = w.E * mpad
    sp = np.full((S, K // 16), 0x38, np.uint8)
    for gg in range(len(r.expert_ids)):
        lo, hi = int(r.row_offsets[gg]), int(r.row_offsets[gg + 1])
        sp[soff[gg]:soff[gg] + hi - lo] = sa[lo:hi]
    dense = run_nv_gemm(r, a, sa, b, sb, es, hint)
    counts = np.diff(r.row_offsets.astype(np.int64))
    g = int(np.argmax(counts))
    cut = int(soff[g]) + int(counts[g]) // 2 + 5
    for S_used, label in ((S, "full"), (cut, "cut")):
        c = Guarded(np.full((T, N), SENT_BF16, np.uint16))
        mxg.mx_grouped_matmul_nvfp4_padded(to_gpu(a), to_gpu(np.ascontiguousarray(sp[:S_used])), to_gpu(soff),
                                           to_gpu(b), to_gpu(sb), to_gpu(es), c.view(torch.bfloat16),
                                           offsets_gpu(r.row_offsets), to_gpu(r.expert_ids.astype(np.int32)), hint)
        torch.cuda.synchronize()
        c.check(f"padded c {label}")
        out = c.numpy()
        covered = np.zeros(T, bool)
        for gg in range(len(r.expert_ids)):
            lo, hi = int(r.row_offsets[gg]), int(r.row_offsets[gg + 1])
            for t in range(lo, hi):
                covered[t] = int(soff[gg]) + t - lo < S_used
        if label == "full":
            assert np.array_equal(out, dense), "padded and dense A scales gave different results"
        else:
            assert 0 < covered.sum() < T
            assert np.all(out[~covered] == SENT_BF16), "rows without scale rows were written"
            assert np.array_equal(out[covered], dense[covered])
