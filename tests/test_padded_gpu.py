"""GPU parity for the padded / slot-strided MX activation-scale layouts: the
padded quantize must match the oracle bit for bit (padding and rows mapped
past the tensor untouched), and the padded GEMM / fused GEMM must equal the
dense ones bit for bit when their A scales are the same bytes moved."""
import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import oracle
import workloads as W
from common import GemmCase, bits, check_gemm_rows, offsets_gpu, to_gpu

pytestmark = pytest.mark.gpu

SENT_BF16 = 0x7FA5


def slot_offsets(r, round_to=128):
    counts = np.diff(r.row_offsets.astype(np.int64))
    mpad = int(max(1, -(-counts.max() // round_to)) * round_to)
    return (r.expert_ids.astype(np.int64) * mpad).astype(np.uint32), mpad


@pytest.mark.parametrize("fmt", [mxg.MXFP8, mxg.MXFP4])
@pytest.mark.parametrize("K", [256, 1024, 7168])
def test_padded_quantize_matches_oracle(fmt, K):
    w = W.WORKLOADS[5].scaled(tokens=48, E=6, masked=1, top_k=4, K=K)
    r = W.routing(w)
    x = bits(W.activations(w, r))
    T = x.shape[0]
    soff, mpad = slot_offsets(r)
    S = w.E * mpad
    qcols = K // 2 if fmt == mxg.MXFP4 else K
    q_ref, s_ref = oracle.quantize_padded(fmt, x, r.row_offsets, soff, S, np.full((T, qcols), 0xA5, np.uint8),
                                          np.full((S, K // 32), 0x5A, np.uint8))
    q = to_gpu(np.full((T, qcols), 0xA5, np.uint8))
    s = to_gpu(np.full((S, K // 32), 0x5A, np.uint8))
    mxg.mx_grouped_quantize_padded(fmt, to_gpu(x.view(np.int16)).view(torch.bfloat16), q, s, to_gpu(soff),
                                   offsets_gpu(r.row_offsets))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(s.cpu().numpy(), s_ref)


def test_padded_quantize_rows_past_the_tensor_are_untouched():
    w = W.WORKLOADS[5].scaled(tokens=32, E=4, masked=0, top_k=4, K=512)
    r = W.routing(w)
    x = bits(W.activations(w, r))
    T, K = x.shape
    soff = r.row_offsets[:-1].astype(np.uint32)
    S = T - 7
    q_ref, s_ref = oracle.quantize_padded(mxg.MXFP4, x, r.row_offsets, soff, S,
                                          np.full((T, K // 2), 0xA5, np.uint8), np.full((S, K // 32), 0x5A, np.uint8))
    q = to_gpu(np.full((T, K // 2), 0xA5, np.uint8))
    s = to_gpu(np.full((S, K // 32), 0x5A, np.uint8))
    mxg.mx_grouped_quantize_padded(mxg.MXFP4, to_gpu(x.view(np.int16)).view(torch.bfloat16), q, s, to_gpu(soff),
                                   offsets_gpu(r.row_offsets))
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref) and np.all(q[S:] == 0xA5)


def padded_case(case: GemmCase, round_to=128):
    soff, mpad = slot_offsets(case.r, round_to)
    S = case.w.E * mpad
    sp = np.full((S, case.w.K // 32), 0x5A, np.uint8)
    for g in range(len(case.ids)):
        lo, hi = int(case.off[g]), int(case.off[g + 1])
        sp[soff[g]:soff[g] + hi - lo] = case.sa[lo:hi]
    return soff, sp


PAD_CASES = {
    # the 192x256 tile with LDS scales, the eight-wave 256x256 MX tile, per-lane scale loads (K % 1024 != 0)
    "mxfp4_k1024": W.WORKLOADS[5].scaled(tokens=96, E=8, masked=1, top_k=4, N=320, K=1024, swiglu=False),
    "mxfp8_tall": W.WORKLOADS[4].scaled(rows=4096, E=8, N=288, K=1024),
    "mxfp4_k608": W.WORKLOADS[5].scaled(tokens=64, E=6, masked=1, top_k=4, N=256, K=608, swiglu=False),
}


@pytest.mark.parametrize("name", list(PAD_CASES))
def test_padded_gemm_equals_dense_and_oracle(name):
    case = GemmCase(PAD_CASES[name])
    soff, sp = padded_case(case)
    inp = case.gpu_inputs()
    T, N = case.T, case.w.N
    hint = int(case.r.counts.max())
    c0 = torch.full((T, N), SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    c1 = torch.full((T, N), SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    mxg.mx_grouped_matmul(case.fmt, c=c0, max_rows_per_group_hint=hint, **inp)
    mxg.mx_grouped_matmul_padded(case.fmt, inp["a_q"], to_gpu(sp), to_gpu(soff), inp["b_q"], inp["b_scales"], c1,
                                 inp["row_offsets"], inp["expert_ids"], hint)
    torch.cuda.synchronize()
    a0 = c0.view(torch.int16).cpu().numpy().view(np.uint16)
    a1 = c1.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(a0, a1), "padded and dense A scales gave different results"
    rows = np.arange(T)
    ref = oracle.gemm_rows_padded(case.fmt, case.a, sp, soff, case.b, case.sb, case.off, case.ids, N, case.w.K, rows)
    cov = ref["group"] >= 0
    check_gemm_rows(a1[cov], {k: v[cov] for k, v in ref.items() if k != "group"}, name)


def test_padded_gemm_skips_tiles_past_the_scale_tensor():
    case = GemmCase(PAD_CASES["mxfp4_k1024"])
    inp = case.gpu_inputs()
    T, N = case.T, case.w.N
    soff = case.off[:-1].astype(np.uint32)
    S = int(case.off[-2])                              # the last group's scale rows are missing
    c = torch.full((T, N), SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    mxg.mx_grouped_matmul_padded(case.fmt, inp["a_q"], to_gpu(np.ascontiguousarray(case.sa[:S])), to_gpu(soff),
                                 inp["b_q"], inp["b_scales"], c, inp["row_offsets"], inp["expert_ids"])
    torch.cuda.synchronize()
    out = c.view(torch.int16).cpu().numpy().view(np.uint16)
    last = slice(int(case.off[-2]), int(case.off[-1]))
    assert np.all(out[last] == SENT_BF16)
    ref = oracle.gemm_rows(case.fmt, case.a, case.sa, case.b, case.sb, case.off, case.ids, N, case.w.K,
                           np.arange(int(case.off[-2])))
    cov = ref["group"] >= 0
    check_gemm_rows(out[:int(case.off[-2])][cov], {k: v[cov] for k, v in ref.items() if k != "group"}, "skip")


def cut_mid_group(case: GemmCase, round_to=128):
    """A slot layout whose scale tensor ends inside the largest group, part
    way into one of its M tiles: rows before the cut are computed, the rest
    of that group and every group whose slot starts later are not."""
    soff, sp = padded_case(case, round_to)
    counts = np.diff(case.off.astype(np.int64))
    g = int(np.argmax(counts))
    assert counts[g] > 40
    S = int(soff[g]) + int(counts[g]) // 2 + 5
    return soff, np.ascontiguousarray(sp[:S]), S


@pytest.mark.parametrize("name", list(PAD_CASES))
@pytest.mark.parametrize("hint", [0, 1 << 20])
def test_padded_gemm_scale_tensor_ends_mid_group(name, hint):
    case = GemmCase(PAD_CASES[name])
    soff, sp, S = cut_mid_group(case)
    inp = case.gpu_inputs()
    T, N = case.T, case.w.N
    c = torch.full((T, N), SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    mxg.mx_grouped_matmul_padded(case.fmt, inp["a_q"], to_gpu(sp), to_gpu(soff), inp["b_q"], inp["b_scales"], c,
                                 inp["row_offsets"], inp["expert_ids"], hint)
    torch.cuda.synchronize()
    out = c.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.gemm_rows_padded(case.fmt, case.a, sp, soff, case.b, case.sb, case.off, case.ids, N, case.w.K,
                                  np.arange(T))
    cov = ref["group"] >= 0
    assert 0 < cov.sum() < T
    assert np.all(out[~cov] == SENT_BF16), "rows without scale rows were written"
    check_gemm_rows(out[cov], {k: v[cov] for k, v in ref.items() if k != "group"}, f"{name} hint={hint}")


@pytest.mark.parametrize("hint", [0, 1 << 20])
def test_padded_fused_swiglu_scale_tensor_ends_mid_group(hint):
    w = W.WORKLOADS[5].scaled(tokens=256, E=8, masked=1, top_k=4, N=256, K=1024)
    case = GemmCase(w)
    soff, sp, S = cut_mid_group(case, round_to=64)
    soff_full, sp_full = padded_case(case, round_to=64)
    inp = case.gpu_inputs()
    T, I = case.T, w.N // 2
    ys = [(torch.full((T, I // 2), 0xA5, dtype=torch.uint8, device="cuda"),
           torch.full((T, I // 32), 0x5A, dtype=torch.uint8, device="cuda")) for _ in range(2)]
    mxg.mx_grouped_matmul_swiglu_padded(case.fmt, inp["a_q"], to_gpu(sp_full), to_gpu(soff_full), inp["b_q"],
                                        inp["b_scales"], ys[0][0], ys[0][1], inp["row_offsets"], inp["expert_ids"],
                                        hint)
    mxg.mx_grouped_matmul_swiglu_padded(case.fmt, inp["a_q"], to_gpu(sp), to_gpu(soff), inp["b_q"],
                                        inp["b_scales"], ys[1][0], ys[1][1], inp["row_offsets"], inp["expert_ids"],
                                        hint)
    torch.cuda.synchronize()
    ref = oracle.gemm_rows_padded(case.fmt, case.a, sp, soff, case.b, case.sb, case.off, case.ids, w.N, w.K,
                                  np.arange(T))
    cov = ref["group"] >= 0
    assert 0 < cov.sum() < T
    full = [y.cpu().numpy() for y in ys[0]]
    cut = [y.cpu().numpy() for y in ys[1]]
    for f, c_ in zip(full, cut):
        assert np.array_equal(f[cov], c_[cov]), "rows with scale rows differ from the uncut layout"
    assert np.all(cut[0][~cov] == 0xA5) and np.all(cut[1][~cov] == 0x5A), "rows without scale rows were written"


def test_padded_fused_swiglu_equals_dense():
    w = W.WORKLOADS[5].scaled(tokens=256, E=8, masked=1, top_k=4, N=256, K=1024)
    case = GemmCase(w)
    soff, sp = padded_case(case, round_to=64)
    inp = case.gpu_inputs()
    T, I = case.T, w.N // 2
    y0 = (torch.zeros((T, I // 2), dtype=torch.uint8, device="cuda"), torch.zeros((T, I // 32), dtype=torch.uint8,
                                                                                   device="cuda"))
    y1 = (torch.zeros((T, I // 2), dtype=torch.uint8, device="cuda"), torch.zeros((T, I // 32), dtype=torch.uint8,
                                                                                   device="cuda"))
    mxg.mx_grouped_matmul_swiglu(case.fmt, inp["a_q"], inp["a_scales"], inp["b_q"], inp["b_scales"], y0[0], y0[1],
                                 inp["row_offsets"], inp["expert_ids"])
    mxg.mx_grouped_matmul_swiglu_padded(case.fmt, inp["a_q"], to_gpu(sp), to_gpu(soff), inp["b_q"], inp["b_scales"],
                                        y1[0], y1[1], inp["row_offsets"], inp["expert_ids"])
    torch.cuda.synchronize()
    assert torch.equal(y0[0], y1[0]) and torch.equal(y0[1], y1[1])
