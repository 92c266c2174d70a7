"""GPU parity: grouped quantize (FP8 rowwise, MXFP8, MXFP4) must match the CPU
oracle bit for bit -- codes and scales -- and leave uncovered rows untouched."""
import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import oracle
import workloads as W
from common import Guarded, SENTINEL, bits, offsets_gpu, oracle_quantize_weights, sentinel_like, to_gpu

pytestmark = pytest.mark.gpu

FMTS = [mxg.FP8_ROWWISE, mxg.MXFP8, mxg.MXFP4]


def run_both(fmt, x_bits: np.ndarray, off: np.ndarray):
    """Quantize the same bf16 rows on both sides, outputs pre-filled with sentinels."""
    T, K = x_bits.shape
    qcols = K // 2 if fmt == mxg.MXFP4 else K
    if fmt == mxg.FP8_ROWWISE:
        s0 = np.full((T,), -3.0, np.float32)
    else:
        s0 = sentinel_like((T, K // 32), value=0x5A)
    q_ref, s_ref = oracle.quantize(fmt, x_bits, off, sentinel_like((T, qcols)), s0.copy())
    x = to_gpu(x_bits.view(np.int16)).view(torch.bfloat16)
    q = Guarded(sentinel_like((T, qcols)))
    s = Guarded(s0.copy())
    mxg.mx_grouped_quantize(fmt, x, q.view(), s.view(), offsets_gpu(off))
    torch.cuda.synchronize()
    q.check("codes")
    s.check("scales")
    return (q.numpy(), s.numpy()), (q_ref, s_ref)


def assert_same(gpu, ref, label):
    (q, s), (qr, sr) = gpu, ref
    bad = np.argwhere(q != qr)
    assert bad.size == 0, f"{label}: {len(bad)} code bytes differ, first at {bad[0]}: gpu {q[tuple(bad[0])]:#x} oracle {qr[tuple(bad[0])]:#x}"
    sb, srb = s.view(np.uint8), sr.view(np.uint8)
    bad = np.argwhere(sb != srb)
    assert bad.size == 0, f"{label}: {len(bad)} scale bytes differ, first at {bad[0]}"


CASES = {
    # (workload, overrides) -- reduced copies of the five workloads (same routing law)
    "tiny": (1, {}),
    "decode": (2, dict(tokens=24)),
    "prefill": (3, dict(tokens=64)),
    "mxfp8": (4, dict(rows=300)),
    "mxfp4": (5, dict(tokens=48)),
}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", list(CASES))
def test_quantize_matches_oracle(fmt, case):
    widx, kw = CASES[case]
    w = W.WORKLOADS[widx].scaled(**kw)
    r = W.routing(w)
    x = bits(W.activations(w, r))
    gpu, ref = run_both(fmt, x, r.row_offsets)
    assert_same(gpu, ref, f"{case} fmt{fmt}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [32, 96, 544, 1056, 2080, 7168, 8192, 8224, 12288])
def test_quantize_row_lengths(fmt, K):
    """Tails of the 512-element wave vector, the register-resident limit, the long-row path and
    (block formats) K segments: 2080 and 7168 are one and two segments with a partial last chunk
    / whole chunks."""
    rng = np.random.default_rng(K + fmt)
    T = 37
    vals = rng.standard_normal((T, K)) * np.exp(rng.uniform(-20, 20, (T, 1)))
    x = oracle.bf16_round_array(vals)
    off = np.array([0, 5, 5, 30, T], np.uint32)
    gpu, ref = run_both(fmt, x, off)
    assert_same(gpu, ref, f"K={K} fmt{fmt}")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_special_values(fmt):
    """Zero rows, signed zeros, bf16 subnormals, the largest bf16, ties and saturation."""
    K = 64
    rows = [
        np.zeros(K),
        np.r_[-0.0, np.zeros(K - 1)],
        np.r_[2.0**-133, -(2.0**-133), 2.0**-126, np.zeros(K - 3)],
        np.r_[3.3895313892515355e38, 1.0, -1e-30, np.zeros(K - 3)],
        np.r_[3.5, -1.0, 0.10009765625, 0.10546875, 2**-15, 1.5 * 2**-16, -(2**-17), np.zeros(K - 7)],
        np.r_[3.90625, 3.0, -0.75, 1.296875, 0.125, 0.375, 1.25, 2.5, np.zeros(K - 8)],
        np.tile([448.0, -464.0, 6.0, -5.0, 13.5, 0.0, -0.0, 1e-20], K // 8),
    ]
    x = oracle.bf16_round_array(np.stack(rows))
    off = np.array([0, len(rows)], np.uint32)
    gpu, ref = run_both(fmt, x, off)
    assert_same(gpu, ref, f"special fmt{fmt}")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_group_coverage(fmt):
    """Uncovered rows, empty groups, an inverted group and offsets past the end."""
    rng = np.random.default_rng(fmt)
    T, K = 40, 128
    x = oracle.bf16_round_array(rng.standard_normal((T, K)))
    for off in ([3, 3, 10, 10, 20],        # rows 0..2 and 20..39 uncovered, empty groups
                [25, 5, 15, 60],           # g0 inverted (skipped), g2 clamped to T
                [0, 0],                    # one empty group
                [7, 9]):                   # a single short group
        gpu, ref = run_both(fmt, x, np.array(off, np.uint32))
        assert_same(gpu, ref, f"coverage {off} fmt{fmt}")


@pytest.mark.parametrize("widx", [2, 3, 4, 5])
def test_quantize_full_size_activations(widx):
    """The full-size activations of each workload, every row, bit for bit."""
    w = W.WORKLOADS[widx]
    r = W.routing(w)
    xg = W.activations(w, r, device="cuda")
    x = bits(xg)
    fmt = w.fmt
    T, K = x.shape
    q_ref, s_ref = oracle.quantize(fmt, x, r.row_offsets)
    q, s = mxg.quantize(fmt, xg, offsets_gpu(r.row_offsets))
    torch.cuda.synchronize()
    assert_same((q.cpu().numpy(), s.cpu().numpy()), (q_ref, s_ref), f"workload {widx}")


@pytest.mark.parametrize("widx", [1, 2, 3, 4, 5])
def test_weight_preparation_full_size(widx):
    """Weights are quantized by the same call (one group of E*N rows): every
    expert of the small workload, four full [N, K] expert slabs of the others
    (rows are independent, so a slab is the same launch on fewer rows)."""
    w = W.WORKLOADS[widx]
    experts = list(range(w.E)) if w.E * w.N * w.K <= 2**28 else [0, 1, w.E // 2, w.E - 1]
    wt = W.weights(w, device="cuda", experts=experts)
    qg, sg = mxg.quantize_weights(w.fmt, wt)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle_quantize_weights(w.fmt, bits(wt))
    assert_same((qg.cpu().numpy(), sg.cpu().numpy()), (q_ref, s_ref), f"weights {widx}")


# ---------------------------------------------------------------- gathered quantize
def run_gather_both(fmt, x_src_bits: np.ndarray, idx: np.ndarray, div: int, off: np.ndarray):
    S, K = x_src_bits.shape
    T = idx.size
    qcols = K // 2 if fmt == mxg.MXFP4 else K
    s0 = np.full((T,), -3.0, np.float32) if fmt == mxg.FP8_ROWWISE else sentinel_like((T, K // 32), value=0x5A)
    q_ref, s_ref = oracle.quantize_gather(fmt, x_src_bits, idx, div, off, sentinel_like((T, qcols)), s0.copy())
    x = to_gpu(x_src_bits.view(np.int16)).view(torch.bfloat16)
    q = to_gpu(sentinel_like((T, qcols)))
    s = to_gpu(s0.copy())
    mxg.mx_grouped_quantize_gather(fmt, x, to_gpu(idx.astype(np.int32)), div, q, s, offsets_gpu(off))
    torch.cuda.synchronize()
    return (q.cpu().numpy(), s.cpu().numpy()), (q_ref, s_ref)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", ["prefill", "mxfp4"])
def test_quantize_gather_matches_oracle(fmt, case):
    """Routed rows read from the token rows through flat slot indices (divisor top_k)."""
    widx, kw = CASES[case]
    w = W.WORKLOADS[widx].scaled(**kw)
    r = W.routing(w)
    xs = bits(W.source_activations(w, r))
    idx = W.slot_indices(r, w.top_k)
    gpu, ref = run_gather_both(fmt, xs, idx, w.top_k, r.row_offsets)
    assert_same(gpu, ref, f"gather {case} fmt={fmt}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [32, 1024, 8704])
def test_quantize_gather_edge_rows(fmt, K):
    """Uncovered rows, negative indices and indices past the source rows are
    left untouched; K = 8704 takes the long-row kernel."""
    rng = np.random.default_rng(K + fmt)
    S, div, T = 19, 3, 70
    xs = oracle.bf16_round_array(rng.standard_normal((S, K)) * np.exp(rng.uniform(-3, 3, (S, 1))))
    idx = rng.integers(0, S * div, T).astype(np.int32)
    idx[[3, 11, 40]] = -7
    idx[[5, 50]] = S * div + 4
    idx[60] = np.iinfo(np.int32).max
    off = np.array([2, 20, 20, 64], np.uint32)  # rows 0-1 and 64.. uncovered
    gpu, ref = run_gather_both(fmt, xs, idx, div, off)
    assert_same(gpu, ref, f"gather edges K={K} fmt={fmt}")


def test_quantize_gather_full_size_prefill():
    """The prefill workload's 65,536 routed rows read straight from its 8192
    token rows, in the benchmark's launch configuration."""
    w = W.WORKLOADS[3]
    r = W.routing(w)
    xs_gpu = W.source_activations(w, r, device="cuda")
    idx = W.slot_indices(r, w.top_k)
    q, s = mxg.quantize_gather(w.fmt, xs_gpu, to_gpu(idx), w.top_k, offsets_gpu(r.row_offsets))
    torch.cuda.synchronize()
    rows = np.unique(np.r_[r.row_offsets[:-1], r.row_offsets[1:] - 1,
                           np.random.default_rng(7).integers(0, r.total_rows, 256)]).astype(np.int64)
    rows = rows[rows < r.total_rows]
    xs = bits(xs_gpu)
    sub_idx = idx[rows]
    q_ref, s_ref = oracle.quantize_gather(w.fmt, xs, sub_idx, w.top_k, np.array([0, rows.size], np.uint32))
    assert np.array_equal(q.cpu().numpy()[rows], q_ref)
    assert np.array_equal(s.cpu().numpy()[rows].view(np.uint8), s_ref.view(np.uint8))


# ---------------------------------------------------------------- token-major (scatter) quantize
def run_scatter_both(fmt, x_tok_bits: np.ndarray, ros: np.ndarray, T: int, off: np.ndarray):
    S, K = x_tok_bits.shape
    qcols = K // 2 if fmt == mxg.MXFP4 else K
    s0 = np.full((T,), -3.0, np.float32) if fmt == mxg.FP8_ROWWISE else sentinel_like((T, K // 32), value=0x5A)
    q_ref, s_ref = oracle.quantize_scatter(fmt, x_tok_bits, ros, T, off, sentinel_like((T, qcols)), s0.copy())
    x = to_gpu(x_tok_bits.view(np.int16)).view(torch.bfloat16)
    q = Guarded(sentinel_like((T, qcols)))
    s = Guarded(s0.copy())
    mxg.mx_grouped_quantize_scatter(fmt, x, to_gpu(ros.astype(np.int32)), q.view(), s.view(), offsets_gpu(off))
    torch.cuda.synchronize()
    q.check("scatter codes")
    s.check("scatter scales")
    return (q.numpy(), s.numpy()), (q_ref, s_ref)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", ["prefill", "mxfp4"])
def test_quantize_scatter_matches_oracle_and_gather(fmt, case):
    """Token rows quantized once and stored to their routed rows through the
    inverse slot map: bit-exact with the oracle, and equal to the gathered
    form on the same routing."""
    widx, kw = CASES[case]
    w = W.WORKLOADS[widx].scaled(**kw)
    r = W.routing(w)
    xs = bits(W.source_activations(w, r))
    ros = W.rows_of_slots(r, w.top_k, xs.shape[0])
    gpu, ref = run_scatter_both(fmt, xs, ros, r.total_rows, r.row_offsets)
    assert_same(gpu, ref, f"scatter {case} fmt={fmt}")
    g_gpu, _ = run_gather_both(fmt, xs, W.slot_indices(r, w.top_k), w.top_k, r.row_offsets)
    assert_same(gpu, g_gpu, f"scatter == gather {case} fmt={fmt}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [32, 1056, 7168])
def test_quantize_scatter_edge_slots(fmt, K):
    """Dropped slots (negative, past the rows), rows no group covers and rows
    no slot names are left untouched; top_k of 1 and 64."""
    rng = np.random.default_rng(K + 10 * fmt)
    for S, top_k in ((23, 3), (3, 64), (40, 1)):
        T = 70
        xs = oracle.bf16_round_array(rng.standard_normal((S, K)) * np.exp(rng.uniform(-3, 3, (S, 1))))
        ros = rng.permutation(max(T, S * top_k))[:S * top_k].astype(np.int32)   # some >= T (dropped)
        ros[rng.integers(0, S * top_k, 3)] = -2
        off = np.array([2, 20, 20, 64], np.uint32)  # rows 0-1 and 64.. uncovered
        gpu, ref = run_scatter_both(fmt, xs, ros, T, off)
        assert_same(gpu, ref, f"scatter edges K={K} fmt={fmt} S={S} top_k={top_k}")


@pytest.mark.parametrize("widx", [3, 5])
def test_quantize_scatter_full_size(widx):
    """The prefill (FP8 rowwise) and fused (MXFP4) workloads at full size, in
    the benchmark's launch configuration: every routed row bit-exact."""
    w = W.WORKLOADS[widx]
    r = W.routing(w)
    xs_gpu = W.source_activations(w, r, device="cuda")
    xs = bits(xs_gpu)
    ros = W.rows_of_slots(r, w.top_k, xs.shape[0])
    T, K = r.total_rows, w.K
    qcols = K // 2 if w.fmt == mxg.MXFP4 else K
    q = torch.zeros((T, qcols), dtype=torch.uint8, device="cuda")
    s = torch.zeros((T,), dtype=torch.float32, device="cuda") if w.fmt == 0 else \
        torch.zeros((T, K // 32), dtype=torch.uint8, device="cuda")
    mxg.mx_grouped_quantize_scatter(w.fmt, xs_gpu, to_gpu(ros), q, s, offsets_gpu(r.row_offsets))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_scatter(w.fmt, xs, ros, T, r.row_offsets)
    assert_same((q.cpu().numpy(), s.cpu().numpy()), (q_ref, s_ref), f"scatter workload {widx}")
