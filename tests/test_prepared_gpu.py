"""GPU parity for the prepared FP8 rowwise weights: the preparation kernel
writes exactly the documented layout (checked byte for byte against a numpy
rearrangement of the same codes), and the grouped GEMM that reads it gives
the oracle's results within the GEMM tolerance and bit-identical results to
the GEMM on the row-major weights, on every reduced FP8 case whose K is a
multiple of 64 (partial M and N tiles, one to fifteen 64-byte stages) and at
the full prefill size.  The prepared path runs 256 x 384 or 256 x 256 tiles,
chosen from the problem's size (the full prefill takes 256 x 384, the reduced
cases 256 x 256); MXG_FP8_TILE forces either, so every reduced case runs
through both, with N = 256 to 1536 (the last 256 x 384 tile of N = 1104 has
336 columns), small launches (every tile split into column halves), a launch
of whole rounds plus a split one, and the full prefill launch (whole tiles
only).  Outputs sit between guard bytes."""
import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import workloads as W
from common import Guarded, GemmCase, check_gemm_rows, sample_rows, to_gpu
from test_gemm_gpu import SENT_BF16, SMALL, check_all_rows, run_gemm

pytestmark = pytest.mark.gpu

FP8_CASES = [n for n, w in SMALL.items() if w.fmt == W.FP8_ROWWISE and w.K % 64 == 0]

# shapes for the 256 x 384 tile beyond the reduced cases above
WIDE = {
    "wide_n1104_partial": W.WORKLOADS[3].scaled(tokens=96, E=16, N=1104, K=512),
    "wide_n768_k64": W.WORKLOADS[3].scaled(tokens=64, E=12, top_k=4, N=768, K=64),
    "wide_n1536_k128": W.WORKLOADS[3].scaled(tokens=128, E=16, N=1536, K=128),
    # last 384-column tile 232 columns wide: its last 16-column load group
    # reaches 8 columns past N (zero rows of the prepared block)
    "wide_n1000": W.WORKLOADS[3].scaled(tokens=64, E=8, top_k=4, N=1000, K=128),
}


def reference_layout(b: np.ndarray) -> np.ndarray:
    """The documented prepared layout, by plain indexing: block (e, nt, s) of
    256 rows x 64 bytes; row r at byte 64 r, its 16-byte position p holding
    piece p ^ ((r >> 2) & 3) of K bytes [64 s, 64 s + 64); rows past N zero."""
    E, N, K = b.shape
    ntn, nst = -(-N // 256), K // 64
    pad = np.zeros((E, ntn * 256, K), np.uint8)
    pad[:, :N] = b
    v = pad.reshape(E, ntn, 256, nst, 4, 16)
    r = np.arange(256)[:, None]
    p = np.arange(4)[None, :]
    src = p ^ ((r >> 2) & 3)
    out = np.empty((E, ntn, nst, 256, 4, 16), np.uint8)
    for s in range(nst):
        out[:, :, s] = v[:, :, r, s, src, :]
    return out.reshape(-1)


@pytest.mark.parametrize("shape", [(3, 96, 128), (2, 512, 192), (1, 300, 64), (4, 256, 1024)])
def test_prepare_writes_the_documented_layout(shape):
    E, N, K = shape
    rng = np.random.default_rng(E * 1000 + N + K)
    b = rng.integers(0, 256, size=shape, dtype=np.uint8)
    n = mxg.prepared_weights_bytes(E, N, K)
    assert n == E * (-(-N // 256)) * 256 * K
    g = Guarded(np.full((n,), 0xEE, np.uint8))
    mxg.mx_prepare_weights_fp8(to_gpu(b), g.view())
    torch.cuda.synchronize()
    g.check("prepared weights")
    assert np.array_equal(g.numpy(), reference_layout(b))


def run_prepared(case: GemmCase):
    inp = case.gpu_inputs()
    bp = mxg.prepare_weights_fp8(inp["b_q"])
    g = Guarded(np.full((case.T, case.w.N), SENT_BF16, np.uint16))
    mxg.mx_grouped_matmul_prepared(inp["a_q"], inp["a_scales"], bp, inp["b_scales"], g.view(torch.bfloat16),
                                   inp["row_offsets"], inp["expert_ids"])
    torch.cuda.synchronize()
    g.check("c, prepared weights")
    return g.numpy()


TILES = ["256x256", "256x384"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("name", FP8_CASES)
def test_prepared_gemm_matches_oracle_and_plain_gemm(name, tile, monkeypatch):
    case = GemmCase(SMALL[name])
    monkeypatch.setenv("MXG_FP8_TILE", tile)
    c = run_prepared(case)
    check_all_rows(case, c, f"{name} prepared {tile}")
    monkeypatch.delenv("MXG_FP8_TILE")
    assert np.array_equal(c, run_gemm(case, hint=1 << 20)), "prepared and row-major weights disagree"
    assert np.array_equal(c, run_gemm(case, hint=0))


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("name", list(WIDE))
def test_wide_shapes_match_oracle_and_plain_gemm(name, tile, monkeypatch):
    case = GemmCase(WIDE[name])
    monkeypatch.setenv("MXG_FP8_TILE", tile)
    c = run_prepared(case)
    check_all_rows(case, c, f"{name} prepared {tile}")
    monkeypatch.setenv("MXG_FP8_TILE", "256x256" if tile == "256x384" else "256x384")
    assert np.array_equal(c, run_gemm(case, hint=1 << 20)), "prepared and row-major weights disagree"


def test_wide_tile_whole_and_split_rounds(monkeypatch):
    """Every token routed to all 8 experts: 8 groups of 14,336 rows, 448 M
    tiles by 2 N tiles of 384 columns (N = 768) = 896 tiles, so on 256
    compute units three whole rounds run and the last 128 tiles split into
    256 column halves.  The size rule picks 256 x 384 here by itself
    (estimated 4 rounds against 6 of 256 x 256); compared with the 256 x 256
    tile on the row-major weights."""
    w = W.WORKLOADS[3].scaled(tokens=14336, E=8, top_k=8, N=768, K=256)
    case = GemmCase(w, gen_device="cuda")
    monkeypatch.delenv("MXG_FP8_TILE", raising=False)
    assert mxg.fp8_tile(len(case.ids), case.T, w.N, w.K, prepared=True) == 384
    c = run_prepared(case)
    monkeypatch.setenv("MXG_FP8_TILE", "256x256")
    assert np.array_equal(c, run_gemm(case, hint=int(case.r.counts.max())))
    rows = sample_rows(case.off, np.random.default_rng(5), per_group_extra=2, extra=16)
    worst, exact = check_gemm_rows(c[rows], case.oracle_rows(rows), "whole and split rounds")
    print(f"whole+split rounds: {rows.size} rows, max |err|/tol = {worst:.3g}, bf16-exact = {exact:.4f}")


def test_prepared_gemm_full_prefill(monkeypatch):
    """The prefill workload at full size (the size rule picks 256 x 384):
    bit-identical to the row-major GEMM through 256 x 256 on every output, and
    within tolerance of the oracle on sampled rows."""
    w = W.WORKLOADS[3]
    case = GemmCase(w, gen_device="cuda")
    monkeypatch.delenv("MXG_FP8_TILE", raising=False)
    assert mxg.fp8_tile(len(case.ids), case.T, w.N, w.K, prepared=True) == 384
    c = run_prepared(case)
    monkeypatch.setenv("MXG_FP8_TILE", "256x256")
    assert np.array_equal(c, run_gemm(case, hint=int(case.r.counts.max())))
    rows = sample_rows(case.off, np.random.default_rng(3), per_group_extra=1, extra=16)
    ref = case.oracle_rows(rows)
    worst, exact = check_gemm_rows(c[rows], ref, "prefill prepared")
    print(f"prefill prepared: {rows.size} rows, max |err|/tol = {worst:.3g}, bf16-exact = {exact:.4f}")


def test_prepared_gemm_no_rows_is_a_no_op():
    case = GemmCase(SMALL["fp8_k64"])
    inp = case.gpu_inputs()
    bp = mxg.prepare_weights_fp8(inp["b_q"])
    c = torch.full((0, case.w.N), 0, dtype=torch.bfloat16, device="cuda")
    off = torch.zeros(len(case.ids) + 1, dtype=torch.int32, device="cuda")
    mxg.mx_grouped_matmul_prepared(inp["a_q"][:0], inp["a_scales"][:0], bp, inp["b_scales"], c, off,
                                   inp["expert_ids"])
    torch.cuda.synchronize()
