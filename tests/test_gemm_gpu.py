"""GPU parity: ragged grouped GEMM (FP8 rowwise, MXFP8, MXFP4) against the CPU
oracle, element by element within |gpu - exact| <= 1e-2 * sum_k |a*b| *
scales + 1 bf16 ulp; uncovered rows must keep their sentinel."""
import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import oracle
import workloads as W
from common import Guarded, GemmCase, check_gemm_rows, sample_rows

pytestmark = pytest.mark.gpu

SENT_BF16 = 0x7FA5  # a NaN pattern no result can produce


def run_gemm(case: GemmCase, N=None, hint=0):
    inp = case.gpu_inputs()
    N = N if N is not None else case.w.N
    g = Guarded(np.full((case.T, N), SENT_BF16, np.uint16))
    mxg.mx_grouped_matmul(case.fmt, c=g.view(torch.bfloat16), max_rows_per_group_hint=hint, **inp)
    torch.cuda.synchronize()
    g.check(f"c, hint {hint}")
    return g.numpy()


def check_all_rows(case: GemmCase, c: np.ndarray, label: str):
    rows = np.arange(case.T)
    ref = case.oracle_rows(rows)
    covered = ref["group"] >= 0
    assert np.all(c[~covered] == SENT_BF16), f"{label}: uncovered rows were written"
    worst, exact = check_gemm_rows(c[covered], {k: v[covered] for k, v in ref.items() if k != "group"}, label)
    print(f"{label}: max |err|/tol = {worst:.3g}, bf16-exact fraction = {exact:.4f}")
    return worst, exact


# Reduced copies of the workloads: several tiles, ragged M tails (group sizes
# not multiples of the tile), N and K not multiples of the tile or stage.
SMALL = {
    "tiny_fp8": W.WORKLOADS[1],
    "decode_fp8": W.WORKLOADS[2].scaled(tokens=32, N=320, K=1056),
    "prefill_fp8": W.WORKLOADS[3].scaled(tokens=160, E=16, N=384, K=1024),
    # FP8 rowwise 64-byte stages: an odd stage count, and one to three stages
    # (the four-slot pipeline's prologue and drain)
    "prefill_fp8_k960": W.WORKLOADS[3].scaled(tokens=160, E=16, N=384, K=960),
    "fp8_k64": W.WORKLOADS[3].scaled(tokens=96, E=8, top_k=3, N=256, K=64),
    "fp8_k128": W.WORKLOADS[3].scaled(tokens=96, E=8, top_k=3, N=256, K=128),
    "fp8_k192": W.WORKLOADS[3].scaled(tokens=96, E=8, top_k=3, N=256, K=192),
    "mxfp8": W.WORKLOADS[4].scaled(rows=700, E=8, N=288, K=608),
    "mxfp4": W.WORKLOADS[5].scaled(tokens=96, E=16, N=256, K=1344),
    "mxfp4_ktail": W.WORKLOADS[5].scaled(tokens=40, E=6, masked=1, top_k=4, N=192, K=800, swiglu=False),
    # K a multiple of 1024: whole stages, MX scales staged through LDS
    "mxfp8_k1024": W.WORKLOADS[4].scaled(rows=700, E=8, N=288, K=1024),
    "mxfp4_k2048": W.WORKLOADS[5].scaled(tokens=96, E=16, N=320, K=2048, swiglu=False),
    # the down-projection after the fused SwiGLU: K = I = 2048, N = hidden = 7168
    "mxfp4_down_proj": W.WORKLOADS[5].scaled(tokens=24, E=8, N=7168, K=2048, swiglu=False),
    # 384+ rows per group on average: the MX formats take the eight-wave 256 x 256 tile
    "mxfp8_tall": W.WORKLOADS[4].scaled(rows=4096, E=8, N=288, K=1024),
    "mxfp4_tall": W.WORKLOADS[5].scaled(tokens=1024, E=8, masked=1, top_k=4, N=320, K=1024, swiglu=False),
}


# The row-count hint selects the tile shape: 0 lets small reduced problems use
# the decode-regime tile, a large hint forces the prefill-regime tile (FP8:
# 256 x 256 or 256 x 384 with eight waves, 64-byte stages when K is a
# multiple of 64, else 256 x 256 with 128-byte stages in two slots; MX:
# 192 x 256 with eight waves when K is a multiple of 1024, else 128 x 256),
# so both code paths see every case, including partial M / N tiles and K
# tails.  Which FP8 256-row tile runs is chosen from the problem's size (the
# reduced cases take 256 x 256); MXG_FP8_TILE forces either one, and
# test_fp8_256_row_tiles_agree runs both.
HINTS = [0, 1 << 20]
FP8_WIDE_CASES = [n for n, w in SMALL.items() if w.fmt == W.FP8_ROWWISE and w.K % 64 == 0 and w.N % 8 == 0]


@pytest.mark.parametrize("hint", HINTS)
@pytest.mark.parametrize("name", list(SMALL))
def test_gemm_matches_oracle_all_rows(name, hint):
    case = GemmCase(SMALL[name])
    c = run_gemm(case, hint=hint)
    worst, exact = check_all_rows(case, c, f"{name} hint={hint}")
    assert exact > 0.9, "most outputs should round to the same bf16 as the exact value"


@pytest.mark.parametrize("name", list(SMALL))
def test_gemm_hint_does_not_change_results(name):
    case = GemmCase(SMALL[name])
    c0 = run_gemm(case, hint=0)
    c1 = run_gemm(case, hint=int(case.r.counts.max()))
    c2 = run_gemm(case, hint=1)
    assert np.array_equal(c0, c1) and np.array_equal(c0, c2)


@pytest.mark.parametrize("widx", [1, 2, 3, 4, 5])
def test_gemm_full_size_sampled_rows(widx):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    computes whole output rows for the first and last row of every group plus
    random rows.  Workload 5 runs here as a plain MXFP4 GEMM with N = 2I."""
    w = W.WORKLOADS[widx]
    case = GemmCase(w, gen_device="cuda")
    c = run_gemm(case)
    rng = np.random.default_rng(widx)
    rows = sample_rows(case.off, rng, per_group_extra=1, extra=32)
    ref = case.oracle_rows(rows)
    assert np.all(ref["group"] >= 0)
    worst, exact = check_gemm_rows(c[rows], ref, f"workload {widx}")
    print(f"workload {widx}: {rows.size} rows, max |err|/tol = {worst:.3g}, bf16-exact = {exact:.4f}")
    # rows beyond the routed total do not exist here; every row is covered
    assert not np.any(c == SENT_BF16)


@pytest.mark.parametrize("fmt", [W.MXFP8, W.MXFP4])
def test_gemm_mx_on_prefill_shape_sampled_rows(fmt):
    """The prefill routing and shape (128 experts, 512 rows per expert on
    average, K = 4096, N = 1536) in the MX formats: the regime of the
    eight-wave MX tile, at full size, sampled rows."""
    w = W.WORKLOADS[3].scaled(fmt=fmt)
    case = GemmCase(w, gen_device="cuda")
    c = run_gemm(case, hint=int(case.r.counts.max()))
    rng = np.random.default_rng(30 + fmt)
    rows = sample_rows(case.off, rng, per_group_extra=1, extra=32)
    ref = case.oracle_rows(rows)
    worst, exact = check_gemm_rows(c[rows], ref, f"prefill shape fmt {fmt}")
    print(f"prefill shape fmt {fmt}: {rows.size} rows, max |err|/tol = {worst:.3g}, bf16-exact = {exact:.4f}")
    assert not np.any(c == SENT_BF16)


@pytest.mark.parametrize("name", FP8_WIDE_CASES)
def test_fp8_256_row_tiles_agree(name, monkeypatch):
    """FP8 rowwise on row-major weights through the 256 x 384 tile (forced) and
    the 256 x 256 tile (forced): bit-identical, and within tolerance of the
    oracle on every row."""
    case = GemmCase(SMALL[name])
    monkeypatch.setenv("MXG_FP8_TILE", "256x384")
    wide = run_gemm(case, hint=1 << 20)
    check_all_rows(case, wide, f"{name} 256x384")
    monkeypatch.setenv("MXG_FP8_TILE", "256x256")
    assert np.array_equal(wide, run_gemm(case, hint=1 << 20)), "256x384 and 256x256 tiles disagree"
