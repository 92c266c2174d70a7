"""Ragged-group edge cases of the grouped GEMM on the GPU, against the oracle:
empty groups, a single group, one-row groups, permuted / repeated / subset
expert ids, out-of-range ids and malformed offsets (skipped, never read out of
bounds), uncovered rows (left untouched) and N / K tails."""
import contextlib
import os

import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import oracle
from common import Guarded, check_gemm_rows, ids_gpu, offsets_gpu, to_gpu

pytestmark = pytest.mark.gpu

SENT = 0x7FA5


def random_operands(rng, fmt, T, E, N, K):
    x = oracle.bf16_round_array(rng.standard_normal((T, K)))
    wt = oracle.bf16_round_array(rng.standard_normal((E * N, K)) * 0.02)
    a, sa = oracle.quantize(fmt, x, np.array([0, T], np.uint32))
    b, sb = oracle.quantize(fmt, wt, np.array([0, E * N], np.uint32))
    b = b.reshape(E, N, -1)
    sb = sb.reshape(E, N) if fmt == 0 else sb.reshape(E, N, K // 32)
    return a, sa, b, sb


@contextlib.contextmanager
def fp8_tile(tile):
    """MXG_FP8_TILE set for the duration (None: the library's own choice)."""
    old = os.environ.get("MXG_FP8_TILE")
    if tile is None:
        os.environ.pop("MXG_FP8_TILE", None)
    else:
        os.environ["MXG_FP8_TILE"] = tile
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("MXG_FP8_TILE", None)
        else:
            os.environ["MXG_FP8_TILE"] = old


def run_case(fmt, a, sa, b, sb, off, ids, N, K):
    """Both tile regimes (hint 0 and a hint that forces the large tile) must
    agree bit for bit and match the oracle; uncovered rows keep the sentinel.
    FP8 rowwise with K % 64 == 0 and N % 8 == 0 also runs the large tile as
    256 x 384 (forced) and the prepared weights under both 256-row tiles."""
    T = a.shape[0]
    runs = [(hint, None, False) for hint in (0, 1 << 20)]
    if fmt == 0 and K % 64 == 0 and N % 8 == 0:
        runs += [(1 << 20, "256x384", False), (0, "256x256", True), (0, "256x384", True)]
    outs = []
    for hint, tile, prepared in runs:
        g = Guarded(np.full((T, N), SENT, np.uint16))
        with fp8_tile(tile):
            if prepared:
                bp = mxg.prepare_weights_fp8(to_gpu(b))
                mxg.mx_grouped_matmul_prepared(to_gpu(a), to_gpu(sa), bp, to_gpu(sb), g.view(torch.bfloat16),
                                               offsets_gpu(off), ids_gpu(ids))
            else:
                mxg.mx_grouped_matmul(fmt, to_gpu(a), to_gpu(sa), to_gpu(b), to_gpu(sb), g.view(torch.bfloat16),
                                      offsets_gpu(off), ids_gpu(ids), hint)
            torch.cuda.synchronize()
        label = f"fmt {fmt} hint {hint} tile {tile or 'chosen'}{' prepared' if prepared else ''}"
        g.check(label)
        outs.append(g.numpy())
        assert np.array_equal(outs[0], outs[-1]), f"{label} disagrees with the first run"
    c = outs[0]
    ref = oracle.gemm_rows(fmt, a, sa, b, sb, off, ids, N, K, np.arange(T))
    cov = ref["group"] >= 0
    assert np.all(c[~cov] == SENT), "a row no valid group covers was written"
    if cov.any():
        check_gemm_rows(c[cov], {k: v[cov] for k, v in ref.items() if k != "group"})
    return cov


GROUPINGS = {
    "empty_groups": ([0, 0, 50, 50, 50, 130, 130], [0, 1, 2, 3, 1, 0]),
    "single_group": ([0, 130], [2]),
    "one_row_groups": ([0, 1, 2, 3, 4, 130], [3, 0, 3, 1, 2]),
    "permuted_and_repeated": ([0, 33, 64, 65, 129, 130], [3, 3, 0, 2, 3]),
    "subset_with_gaps": ([5, 40, 40, 90], [1, 1, 2]),           # rows 0..4 and 90.. uncovered
    "out_of_range_ids": ([0, 40, 80, 130], [4, -1, 1]),         # groups 0 and 1 skipped
    "inverted_and_past_end": ([60, 20, 100, 500], [0, 1, 2]),   # g0 inverted; g2 clamped to T
    "all_empty": ([7, 7, 7], [0, 1]),
}


# K = 288 has a partial last stage; K = 512 does not; with K = 1024 the MX
# formats also stage their scales through LDS (large-tile hint of run_case).
@pytest.mark.parametrize("K", [288, 512, 1024])
@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("name", list(GROUPINGS))
def test_groupings(fmt, name, K):
    rng = np.random.default_rng(len(name) * 7 + fmt + K)
    T, E, N = 130, 4, 200
    a, sa, b, sb = random_operands(rng, fmt, T, E, N, K)
    off, ids = GROUPINGS[name]
    run_case(fmt, a, sa, b, sb, np.array(off, np.uint32), np.array(ids, np.int32), N, K)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("N,K", [(32, 32), (96, 64), (129, 160), (1000, 96), (1000, 128), (300, 512), (300, 1024),
                                 (40, 3072)])
def test_shape_tails(fmt, N, K):
    rng = np.random.default_rng(N * K + fmt)
    T, E = 77, 3
    a, sa, b, sb = random_operands(rng, fmt, T, E, N, K)
    run_case(fmt, a, sa, b, sb, np.array([0, 20, 21, 77], np.uint32), np.array([2, 0, 1], np.int32), N, K)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("spread", ["sparse", "skewed"])
def test_many_groups(fmt, spread):
    """The largest group count, 1024 groups.  Sparse: 600 rows over all of
    them (most groups empty or a row or two).  Skewed: 3000 rows drawn with
    weights 1/k^1.2 over a shuffled group order (437 non-empty groups, the
    largest 707 rows, so a few span several 256-row tiles), N = 400 and
    K = 1024: every tile regime has more than one column tile (the 256 x 384
    tile a partial last one), the MX formats stage their scales through LDS,
    and FP8 also runs the 256 x 384 and prepared-weight tiles (run_case)."""
    rng = np.random.default_rng(99 if spread == "sparse" else 100)
    G, E = 1024, 8
    if spread == "sparse":
        T, N, K = 600, 64, 64
        counts = rng.multinomial(T, np.ones(G) / G)
    else:
        T, N, K = 3000, 400, 1024
        p = 1.0 / np.arange(1, G + 1) ** 1.2
        rng.shuffle(p)
        counts = rng.multinomial(T, p / p.sum())
    off = np.r_[0, np.cumsum(counts)].astype(np.uint32)
    ids = rng.integers(0, E, G).astype(np.int32)
    a, sa, b, sb = random_operands(rng, fmt, T, E, N, K)
    cov = run_case(fmt, a, sa, b, sb, off, ids, N, K)
    assert cov.all()


def test_zero_rows_is_a_no_op():
    e = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    c = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((1, 32, 64), dtype=torch.uint8, device="cuda")
    mxg.mx_grouped_matmul(0, e, torch.empty((0,), device="cuda"), b, torch.zeros((1, 32), device="cuda"), c,
                          offsets_gpu(np.array([0, 0], np.uint32)), ids_gpu(np.array([0], np.int32)))
    torch.cuda.synchronize()
