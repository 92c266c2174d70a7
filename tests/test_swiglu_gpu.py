"""GPU parity for the gated activation + MXFP4 requant, standalone and fused.

* mx_silu_quantize vs the oracle on the same bf16 gate/up input: bit-exact,
  except at elements whose fp64 y lies within 2^-20 (relative) of a bf16
  rounding boundary ("fragile": the GPU evaluates silu in fp32).
* mx_grouped_matmul_swiglu vs mx_grouped_matmul + mx_silu_quantize (both on
  the GPU): byte for byte, as the pages state for the fused kernel.
* mx_grouped_matmul_swiglu vs the oracle's fused path: every scale and code
  must be reachable from gate/up values inside the GEMM tolerance, and nearly
  all bytes equal the oracle's own rounding.
"""
import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import oracle
import workloads as W
from common import Guarded, GemmCase, check_swiglu_interval, offsets_gpu, sample_rows, to_gpu

pytestmark = pytest.mark.gpu


def fragile_mask(y64: np.ndarray, rel=2.0**-20) -> np.ndarray:
    lo = oracle.bf16_round_array(y64 * (1 - rel))
    hi = oracle.bf16_round_array(y64 * (1 + rel))
    return lo != hi


def check_silu_requant(yq, ys, yq_ref, ys_ref, y64):
    """Exact match, with the fragile-element allowance described above."""
    n, I = y64.shape
    frag = fragile_mask(y64)
    frag_blk = frag.reshape(n, I // 32, 32).any(axis=2)
    assert np.array_equal(ys[~frag_blk], ys_ref[~frag_blk]), "block scales differ in non-fragile blocks"
    nib = np.stack([yq & 0xF, yq >> 4], axis=-1).reshape(n, I)
    nib_ref = np.stack([yq_ref & 0xF, yq_ref >> 4], axis=-1).reshape(n, I)
    same_scale = np.repeat(ys == ys_ref, 32, axis=1)
    strict = same_scale & ~np.repeat(frag_blk, 32, axis=1)
    assert np.array_equal(nib[strict], nib_ref[strict]), "codes differ in non-fragile blocks"
    return float(frag.mean())


@pytest.mark.parametrize("I,T", [(32, 17), (2048, 96), (96, 300)])
def test_silu_quantize_matches_oracle(I, T):
    rng = np.random.default_rng(I + T)
    # gate/up values spanning silu's regimes, including exact zeros and ties
    vals = rng.standard_normal((T, 2 * I)) * np.exp(rng.uniform(-6, 4, (T, 1)))
    vals[0, :8] = [0.0, 5.0, -0.0, 3.0, 1.0, 2.0, -20.0, 4.0]
    h = oracle.bf16_round_array(vals)
    off = np.array([0, 3, 3, T - 4], np.uint32)  # last 4 rows uncovered
    yq_ref, ys_ref, y64 = oracle.silu_requant(h, off, np.full((T, I // 2), 0xA5, np.uint8),
                                              np.full((T, I // 32), 0x5A, np.uint8), want_y64=True)
    hg = to_gpu(h.view(np.int16)).view(torch.bfloat16)
    yq = torch.full((T, I // 2), 0xA5, dtype=torch.uint8, device="cuda")
    ys = torch.full((T, I // 32), 0x5A, dtype=torch.uint8, device="cuda")
    mxg.mx_silu_quantize(hg, yq, ys, offsets_gpu(off))
    yq, ys = yq.cpu().numpy(), ys.cpu().numpy()
    cov = np.zeros(T, bool)
    cov[:T - 4] = True
    assert np.all(yq[~cov] == 0xA5) and np.all(ys[~cov] == 0x5A)
    frac = check_silu_requant(yq[cov], ys[cov], yq_ref[cov], ys_ref[cov], y64[cov])
    print(f"fragile fraction {frac:.2e}")


FUSED = {
    "small_mxfp4": W.WORKLOADS[5].scaled(tokens=96, E=16, N=256, K=1344),
    "small_mxfp8": W.WORKLOADS[5].scaled(tokens=64, E=8, N=192, K=640, fmt=W.MXFP8),
    "small_mxfp4_k1024": W.WORKLOADS[5].scaled(tokens=96, E=16, N=384, K=1024),
    # 384+ rows per group on average: the eight-wave 256 x 256 MX tile
    "tall_mxfp4": W.WORKLOADS[5].scaled(tokens=1024, E=8, masked=1, top_k=4, N=320, K=1024),
    "tall_mxfp8": W.WORKLOADS[5].scaled(tokens=1024, E=8, masked=1, top_k=4, N=256, K=1024, fmt=W.MXFP8),
}


def run_fused_and_chained(case: GemmCase, hint: int = 0):
    inp = case.gpu_inputs()
    T, I = case.T, case.w.N // 2
    gq = Guarded(np.full((T, I // 2), 0xA5, np.uint8))
    gs = Guarded(np.full((T, I // 32), 0x5A, np.uint8))
    yq, ys = gq.view(), gs.view()
    mxg.mx_grouped_matmul_swiglu(case.fmt, inp["a_q"], inp["a_scales"], inp["b_q"], inp["b_scales"], yq, ys,
                                 inp["row_offsets"], inp["expert_ids"], hint)
    c = torch.zeros((T, 2 * I), dtype=torch.bfloat16, device="cuda")
    mxg.mx_grouped_matmul(case.fmt, c=c, max_rows_per_group_hint=hint, **inp)
    yq2 = torch.full((T, I // 2), 0xA5, dtype=torch.uint8, device="cuda")
    ys2 = torch.full((T, I // 32), 0x5A, dtype=torch.uint8, device="cuda")
    mxg.mx_silu_quantize(c, yq2, ys2, inp["row_offsets"])
    torch.cuda.synchronize()
    gq.check("fused codes")
    gs.check("fused scales")
    return (yq.cpu().numpy(), ys.cpu().numpy()), (yq2.cpu().numpy(), ys2.cpu().numpy())


def check_against_oracle(case: GemmCase, yq, ys, rows):
    ref = oracle.gemm_swiglu_rows(case.fmt, case.a, case.sa, case.b, case.sb, case.off, case.ids, case.w.N // 2,
                                  case.w.K, rows)
    assert np.all(ref["group"] >= 0)
    check_swiglu_interval(yq[rows], ys[rows], ref["gu_exact"], ref["gu_bound"])
    code_eq = float(np.mean(yq[rows] == ref["yq"]))
    scale_eq = float(np.mean(ys[rows] == ref["ys"]))
    print(f"equal to the oracle's rounding: codes {code_eq:.4f}, scales {scale_eq:.4f}")
    assert code_eq > 0.98 and scale_eq > 0.98


@pytest.mark.parametrize("hint", [0, 1 << 20])
@pytest.mark.parametrize("name", list(FUSED))
def test_fused_equals_chained_and_oracle(name, hint):
    case = GemmCase(FUSED[name])
    (yq, ys), (yq2, ys2) = run_fused_and_chained(case, hint)
    assert np.array_equal(yq, yq2) and np.array_equal(ys, ys2), "fused and chained paths differ"
    check_against_oracle(case, yq, ys, np.arange(case.T))


def test_fused_full_size_sampled_rows():
    w = W.WORKLOADS[5]
    case = GemmCase(w, gen_device="cuda")
    (yq, ys), (yq2, ys2) = run_fused_and_chained(case)
    assert np.array_equal(yq, yq2) and np.array_equal(ys, ys2), "fused and chained paths differ"
    rows = sample_rows(case.off, np.random.default_rng(5), per_group_extra=1, extra=16)
    check_against_oracle(case, yq, ys, rows)


# Sparse and malformed routings (as in the GEMM's ragged suite): the fused
# kernel writes exactly the rows a valid group covers -- groups with an id
# outside [0, E) or inverted offsets are skipped, offsets past the end are
# clamped to T, rows no group covers keep their bytes.
FUSED_GROUPINGS = {
    "empty_groups": ([0, 0, 50, 50, 50, 130, 130], [0, 1, 2, 3, 1, 0]),
    "subset_with_gaps": ([5, 40, 40, 90], [1, 1, 2]),
    "out_of_range_ids": ([0, 40, 80, 130], [4, -1, 1]),
    "inverted_and_past_end": ([60, 20, 100, 500], [0, 1, 2]),
}


@pytest.mark.parametrize("hint", [0, 1 << 20])
@pytest.mark.parametrize("K", [640, 1024])
@pytest.mark.parametrize("fmt", [W.MXFP8, W.MXFP4])
@pytest.mark.parametrize("name", list(FUSED_GROUPINGS))
def test_fused_sparse_and_malformed_routing(name, fmt, K, hint):
    """K = 640 loads the scales per lane, K = 1024 stages them through LDS;
    hint 0 runs the small-group tile, the large hint the large one.  On the
    covered rows the fused result equals the chained GEMM + activation byte
    for byte and is reachable from the oracle's gate/up intervals."""
    from test_ragged_gpu import random_operands

    rng = np.random.default_rng(len(name) * 31 + fmt * 7 + K)
    T, E, N = 130, 4, 256
    I = N // 2
    a, sa, b, sb = random_operands(rng, fmt, T, E, N, K)
    off = np.array(FUSED_GROUPINGS[name][0], np.uint32)
    ids = np.array(FUSED_GROUPINGS[name][1], np.int32)
    off_d, ids_d = offsets_gpu(off), torch.from_numpy(ids).cuda()
    gq = Guarded(np.full((T, I // 2), 0xA5, np.uint8))
    gs = Guarded(np.full((T, I // 32), 0x5A, np.uint8))
    mxg.mx_grouped_matmul_swiglu(fmt, to_gpu(a), to_gpu(sa), to_gpu(b), to_gpu(sb), gq.view(), gs.view(), off_d,
                                 ids_d, hint)
    c = torch.zeros((T, N), dtype=torch.bfloat16, device="cuda")
    mxg.mx_grouped_matmul(fmt, to_gpu(a), to_gpu(sa), to_gpu(b), to_gpu(sb), c, off_d, ids_d, hint)
    yq2 = torch.full((T, I // 2), 0xA5, dtype=torch.uint8, device="cuda")
    ys2 = torch.full((T, I // 32), 0x5A, dtype=torch.uint8, device="cuda")
    mxg.mx_silu_quantize(c, yq2, ys2, off_d)
    torch.cuda.synchronize()
    gq.check("fused codes")
    gs.check("fused scales")
    yq, ys = gq.numpy(), gs.numpy()
    ref = oracle.gemm_swiglu_rows(fmt, a, sa, b, sb, off, ids, I, K, np.arange(T))
    cov = ref["group"] >= 0
    assert np.all(yq[~cov] == 0xA5) and np.all(ys[~cov] == 0x5A), "a row no valid group covers was written"
    assert np.array_equal(yq[cov], yq2.cpu().numpy()[cov]) and np.array_equal(ys[cov], ys2.cpu().numpy()[cov]), \
        "fused and chained paths differ on covered rows"
    if cov.any():
        check_swiglu_interval(yq[cov], ys[cov], ref["gu_exact"][cov], ref["gu_bound"][cov])
