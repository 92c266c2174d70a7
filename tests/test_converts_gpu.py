"""Exhaustive GPU checks of the hardware converts the kernels rely on, each
driven through a public entry point and compared bit for bit with the oracle
(OCP MX v1.0 encoders with round-to-nearest-even and saturation; bf16 RNE):

* the e4m3 and e2m1 converts of the MX quantize: every finite bf16 value
  that can share a block with a planted block maximum, for every shared
  exponent the maximum can force (every X from -127 to the largest a finite
  bf16 maximum reaches);
* the FP8-rowwise quotient x / scale and its e4m3 convert: for row maxima in
  every bf16 binade (five mantissas each, subnormal maxima included), every
  bf16 value from 21 binades below the maximum up to it, both signs;
* the fp32 -> bf16 convert (v_cvt_pk_bf16_f32): through mx_moe_combine with
  one slot per token, a unit routed row and fp32 router weights at every
  fp32 exponent, with low halves at, and one unit either side of, the
  rounding tie.
"""
import numpy as np
import pytest
import torch

import fp4_grouped_gemm_quantize_amd as mxg
import oracle
from common import to_gpu

pytestmark = pytest.mark.gpu


def bf16_max_with_floor_log2(E: int) -> int:
    """Bits of the largest positive bf16 value v with floor(log2 v) = E
    (E from -133 to 127)."""
    if E >= -126:
        return ((E + 127) << 7) | 0x7F
    # subnormal: value = m * 2^-133, floor(log2) = -133 + msb(m)
    msb = E + 133
    return (1 << (msb + 1)) - 1


def mx_sweep_rows(emax: int, K: int = 7168):
    """Blocks of 32: element 0 is the planted maximum of binade E, elements
    1..31 are consecutive entries of the list of every bf16 value whose
    magnitude does not exceed it (both signs).  Returns bf16 bits [rows, K]."""
    blocks = []
    for E in range(-133, 128):
        X = max(-127, min(127, E - emax))
        if E - emax > 127:
            continue
        amax = bf16_max_with_floor_log2(E)
        mags = np.arange(0, amax + 1, dtype=np.uint32)
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        pad = (-vals.size) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        blk = np.concatenate([np.full((vals.shape[0], 1), amax, np.uint16), vals], axis=1)
        blocks.append(blk)
        assert X >= -127
    blk = np.concatenate(blocks)
    per_row = K // 32
    pad = (-blk.shape[0]) % per_row
    blk = np.concatenate([blk, np.zeros((pad, 32), np.uint16)])
    return blk.reshape(-1, K)


def run_quantize(fmt: int, x_bits: np.ndarray):
    T, K = x_bits.shape
    off = np.array([0, T], np.uint32)
    x = to_gpu(x_bits.view(np.int16)).view(torch.bfloat16)
    q, s = mxg.quantize(fmt, x, to_gpu(off.view(np.int32)))
    torch.cuda.synchronize()
    return off, q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("fmt,emax", [(mxg.MXFP8, 8), (mxg.MXFP4, 2)])
def test_mx_quantize_every_bf16_at_every_shared_exponent(fmt, emax):
    x = mx_sweep_rows(emax)
    off, q, s = run_quantize(fmt, x)
    q_ref, s_ref = oracle.quantize(fmt, x, off)
    assert np.array_equal(s, s_ref), "block scales"
    bad = np.argwhere(q != q_ref)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:4].tolist()}"
    # every shared exponent the planted maxima can force was exercised
    forced = np.unique(s_ref)
    assert forced.min() == 0 and forced.max() == 254 - emax
    assert forced.size == 254 - emax + 1


def rowwise_sweep_rows():
    """One row per maximum: element 0 is the maximum, then every bf16 value
    with magnitude in [2^(E-21), maximum] of both signs (and zeros to pad)."""
    rows = []
    for E in range(-133, 128):
        top = bf16_max_with_floor_log2(E)
        if E >= -126:
            tops = [((E + 127) << 7) | m for m in (0x00, 0x01, 0x40, 0x55, 0x7F)]
        else:
            tops = sorted({top, (top + 1) // 2 + (top > 1)})
        for amax in tops:
            lo_E = E - 21
            lo = 0 if lo_E < -133 else bf16_max_with_floor_log2(lo_E - 1) + 1 if lo_E > -133 else 1
            mags = np.arange(lo, amax + 1, dtype=np.uint32)
            rows.append(np.concatenate([[amax], mags, mags | 0x8000]).astype(np.uint16))
    K = max(r.size for r in rows)
    K += (-K) % 32
    x = np.zeros((len(rows), K), np.uint16)
    for i, r in enumerate(rows):
        x[i, :r.size] = r
    return x


def test_rowwise_quantize_every_bf16_near_every_amax():
    x = rowwise_sweep_rows()
    off, q, s = run_quantize(mxg.FP8_ROWWISE, x)
    q_ref, s_ref = oracle.quantize(mxg.FP8_ROWWISE, x, off)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), "row scales"
    bad = np.argwhere(q != q_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}"


def fp32_tie_sweep() -> np.ndarray:
    """fp32 values at every exponent (subnormals included) whose low 16 bits
    sit at, or one unit either side of, the bf16 rounding tie, or at the ends
    of the range, for several bf16 mantissas; both signs."""
    exps = np.arange(0, 255, dtype=np.uint32)
    mants = np.array([0x00, 0x01, 0x3F, 0x40, 0x7E, 0x7F], np.uint32)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = (exps[:, None, None] << 23) | (mants[None, :, None] << 16) | lows[None, None, :]
    bits = bits.reshape(-1)
    bits = np.concatenate([bits, bits | 0x80000000])
    return bits.view(np.float32)


def test_bf16_rounding_of_fp32_through_combine():
    w = fp32_tie_sweep()
    n, H = w.size, 8
    y = np.full((1, H), 0x3F80, np.uint16)           # a routed row of ones
    ros = np.zeros(n, np.int32)
    ref = oracle.combine(y, ros, w, n)["out"]
    out = mxg.moe_combine(to_gpu(y.view(np.int16)).view(torch.bfloat16), to_gpu(ros), to_gpu(w), n)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} outputs differ, e.g. w bits {w.view(np.uint32)[bad[:4, 0]].tolist()}"
