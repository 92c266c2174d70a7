"""MXG_VALIDATE on the GPU: with it set, malformed routing metadata in device
memory is refused before any launch (outputs untouched, the first violation
named); well-formed routing runs unchanged; without it, malformed routing is
handled as the header describes (no error)."""
import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import workloads as W
from common import GemmCase, offsets_gpu, to_gpu

pytestmark = pytest.mark.gpu

SENT_BF16 = 0x7FA5


def gemm_into(case, off, ids):
    inp = case.gpu_inputs()
    inp["row_offsets"], inp["expert_ids"] = off, ids
    c = torch.full((case.T, case.w.N), SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    mxg.mx_grouped_matmul(case.fmt, c=c, **inp)
    torch.cuda.synchronize()
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", [0, 2])
def test_validate_refuses_malformed_routing(monkeypatch, fmt):
    w = W.WORKLOADS[3].scaled(tokens=64, E=8, top_k=3, N=256, K=256, fmt=fmt)
    case = GemmCase(w)
    good_off, good_ids = case.off.astype(np.uint32), case.ids.astype(np.int32)
    bad = {
        "decreasing": (np.r_[good_off[:3], good_off[2] - 1, good_off[4:]].astype(np.uint32), good_ids),
        "past_total_rows": (np.r_[good_off[:-1], case.T + 5].astype(np.uint32), good_ids),
        "expert_out_of_range": (good_off, np.r_[good_ids[:-1], w.E].astype(np.int32)),
    }
    monkeypatch.setenv("MXG_VALIDATE", "1")
    ref = gemm_into(case, offsets_gpu(good_off), to_gpu(good_ids))
    assert mxg.validation_message() == ""
    for name, (off, ids) in bad.items():
        with pytest.raises(mxg.MxgError) as e:
            gemm_into(case, offsets_gpu(off), to_gpu(ids))
        assert e.value.status == mxg.ERROR_INVALID_VALUE, name
        assert mxg.validation_message(), name
    # the refused calls launched nothing: a fresh output stays all sentinel
    c = torch.full((case.T, case.w.N), SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    inp = case.gpu_inputs()
    inp["row_offsets"] = offsets_gpu(bad["decreasing"][0])
    with pytest.raises(mxg.MxgError):
        mxg.mx_grouped_matmul(case.fmt, c=c, **inp)
    torch.cuda.synchronize()
    assert np.all(c.view(torch.int16).cpu().numpy().view(np.uint16) == SENT_BF16)
    # without MXG_VALIDATE the same malformed routing is handled, not refused
    monkeypatch.delenv("MXG_VALIDATE")
    out = gemm_into(case, offsets_gpu(bad["expert_out_of_range"][0]), to_gpu(bad["expert_out_of_range"][1]))
    last = slice(int(good_off[-2]), int(good_off[-1]))
    assert np.all(out[last] == SENT_BF16)              # the group with a bad expert id is skipped
    assert np.array_equal(out[:int(good_off[-2])], ref[:int(good_off[-2])])


def test_validate_quantize(monkeypatch):
    x = torch.randn(64, 128, device="cuda").to(torch.bfloat16)
    q = torch.zeros((64, 128), dtype=torch.uint8, device="cuda")
    s = torch.zeros((64,), dtype=torch.float32, device="cuda")
    monkeypatch.setenv("MXG_VALIDATE", "1")
    mxg.mx_grouped_quantize(0, x, q, s, offsets_gpu(np.array([0, 10, 64], np.uint32)))
    with pytest.raises(mxg.MxgError):
        mxg.mx_grouped_quantize(0, x, q, s, offsets_gpu(np.array([0, 30, 20, 64], np.uint32)))
    assert "below" in mxg.validation_message()
