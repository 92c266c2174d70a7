"""GPU parity for the MoE combine (mx_moe_combine) against the oracle:
|gpu - exact| <= 1/2 bf16 ulp(exact) + (top_k + 1) * 2^-23 * sum_k |w * y|
(the kernel sums in fp32, one fused multiply-add per slot, and rounds once),
dropped slots contribute nothing, every output row is written."""
import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import oracle
import workloads as W
from common import Guarded, to_gpu

pytestmark = pytest.mark.gpu


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -133.0)  # bf16 subnormal spacing 2^-133
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def check_combine(out_bits: np.ndarray, ref: dict, top_k: int):
    got = oracle.bf16_value_array(out_bits)
    e, b = ref["exact"], ref["bound"]
    tol = 0.5 * bf16_ulp(e) + (top_k + 1) * 2.0 ** -23 * b
    err = np.abs(got - e)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, f"{len(bad)} outputs out of tolerance, first {tuple(bad[0])}: gpu {got[tuple(bad[0])]} exact {e[tuple(bad[0])]}"
    return float(np.mean(out_bits == ref["out"]))


def run(y_bits, ros, w, ntok):
    y = to_gpu(y_bits.view(np.int16)).view(torch.bfloat16)
    g = Guarded(np.full((ntok, y_bits.shape[1]), 0x7FA5, np.uint16))
    out = g.view(torch.bfloat16)
    mxg.mx_moe_combine(y, to_gpu(ros.astype(np.int32)), to_gpu(w.astype(np.float32)), out)
    torch.cuda.synchronize()
    g.check("combine out")
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("H", [8, 1000, 4104])
def test_combine_routed_rows(H):
    """Top-8 routing of a reduced MXFP4 workload: every token's slots, router
    weights from a softmax, a few slots dropped."""
    w = W.WORKLOADS[5].scaled(tokens=96, E=16)
    r = W.routing(w)
    ros = W.rows_of_slots(r, w.top_k, w.tokens)
    ros[[5, 77, 300]] = -1                      # dropped slots
    ros[[9]] = r.total_rows + 3                 # a row past the end: also dropped
    wt = W.router_weights(w, w.tokens)
    rng = np.random.default_rng(H)
    y = oracle.bf16_round_array(rng.standard_normal((r.total_rows, H)) * np.exp(rng.uniform(-4, 4, (r.total_rows, 1))))
    out = run(y, ros, wt, w.tokens)
    ref = oracle.combine(y, ros, wt, w.tokens)
    eq = check_combine(out, ref, w.top_k)
    print(f"H={H}: bit-equal to the oracle's rounding {eq:.4f}")
    assert eq > 0.99


def test_combine_many_slots_and_empty_tokens():
    """top_k above one wave's worth of slots, and tokens with no live slot."""
    rng = np.random.default_rng(11)
    T, H, ntok, k = 300, 64, 9, 70
    y = oracle.bf16_round_array(rng.standard_normal((T, H)))
    ros = rng.integers(0, T, ntok * k).astype(np.int32)
    ros[2 * k:3 * k] = -1                      # token 2: nothing live
    wt = rng.standard_normal(ntok * k).astype(np.float32)
    out = run(y, ros, wt, ntok)
    ref = oracle.combine(y, ros, wt, ntok)
    check_combine(out, ref, k)
    assert np.all(out[2] == 0)


def test_combine_zero_tokens_is_a_no_op():
    y = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((0, 16), dtype=torch.bfloat16, device="cuda")
    mxg.mx_moe_combine(y, torch.zeros(0, dtype=torch.int32, device="cuda"),
                       torch.zeros(0, dtype=torch.float32, device="cuda"), out)
    torch.cuda.synchronize()
