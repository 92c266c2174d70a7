"""The C ABI boundary, on the CPU: the library loads, exports every entry point
include/mxg.h declares, and rejects bad arguments with the documented status
before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import fp4_grouped_gemm_quantize_amd as mxg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxg.h")



def test_library_is_built():
    """The boundary tests need the built library; a missing one is a failure
    (build it with `python -m fp4_grouped_gemm_quantize_amd.build`), never a skip."""
    assert os.path.exists(mxg.LIB_PATH), f"libmxg.so not built at {mxg.LIB_PATH}"


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(mxg.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = mxg.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    assert mxg.status_string(0) == "MXG_SUCCESS"
    for s in (1, 2, 3):
        assert mxg.status_string(s).startswith("MXG_ERROR")
    assert "unknown" in mxg.status_string(99)


P = ctypes.c_void_p
FAKE = P(0x10000)      # never dereferenced: validation fails before any launch
FAKE_ODD = P(0x10001)  # misaligned


def q(fmt=0, x=FAKE, qq=FAKE, s=FAKE, off=FAKE, ids=None, G=1, T=4, K=64):
    return mxg.lib().mx_grouped_quantize(fmt, x, qq, s, off, ids, G, T, K, None)


def test_quantize_argument_errors():
    assert q(x=None) == mxg.ERROR_INVALID_VALUE
    assert q(qq=None) == mxg.ERROR_INVALID_VALUE
    assert q(s=None) == mxg.ERROR_INVALID_VALUE
    assert q(off=None) == mxg.ERROR_INVALID_VALUE
    assert q(fmt=3) == mxg.ERROR_INVALID_VALUE
    assert q(fmt=-1) == mxg.ERROR_INVALID_VALUE
    assert q(K=0) == mxg.ERROR_INVALID_VALUE
    assert q(T=-1) == mxg.ERROR_INVALID_VALUE
    assert q(G=-1) == mxg.ERROR_INVALID_VALUE
    assert q(x=FAKE_ODD) == mxg.ERROR_INVALID_VALUE
    assert q(K=48) == mxg.ERROR_NOT_SUPPORTED
    assert q(G=1025) == mxg.ERROR_NOT_SUPPORTED
    # nothing to do: returns success without launching
    assert q(T=0) == mxg.SUCCESS
    assert q(G=0) == mxg.SUCCESS


def qg(fmt=0, x=FAKE, S=8, idx=FAKE, div=2, qq=FAKE, s=FAKE, off=FAKE, ids=None, G=1, T=4, K=64):
    return mxg.lib().mx_grouped_quantize_gather(fmt, x, S, idx, div, qq, s, off, ids, G, T, K, None)


def test_quantize_gather_argument_errors():
    assert qg(idx=None) == mxg.ERROR_INVALID_VALUE
    assert qg(x=None) == mxg.ERROR_INVALID_VALUE
    assert qg(qq=None) == mxg.ERROR_INVALID_VALUE
    assert qg(s=None) == mxg.ERROR_INVALID_VALUE
    assert qg(off=None) == mxg.ERROR_INVALID_VALUE
    assert qg(div=0) == mxg.ERROR_INVALID_VALUE
    assert qg(div=-2) == mxg.ERROR_INVALID_VALUE
    assert qg(S=-1) == mxg.ERROR_INVALID_VALUE
    assert qg(fmt=3) == mxg.ERROR_INVALID_VALUE
    assert qg(idx=FAKE_ODD) == mxg.ERROR_INVALID_VALUE
    assert qg(x=FAKE_ODD) == mxg.ERROR_INVALID_VALUE
    assert qg(K=48) == mxg.ERROR_NOT_SUPPORTED
    assert qg(G=1025) == mxg.ERROR_NOT_SUPPORTED
    assert qg(T=0) == mxg.SUCCESS
    assert qg(G=0) == mxg.SUCCESS


def cb(y=FAKE, T=8, H=64, ros=FAKE, w=FAKE, ntok=2, k=4, out=FAKE):
    return mxg.lib().mx_moe_combine(y, T, H, ros, w, ntok, k, out, None)


def test_combine_argument_errors():
    assert cb(ros=None) == mxg.ERROR_INVALID_VALUE
    assert cb(w=None) == mxg.ERROR_INVALID_VALUE
    assert cb(out=None) == mxg.ERROR_INVALID_VALUE
    assert cb(y=None) == mxg.ERROR_INVALID_VALUE
    assert cb(H=0) == mxg.ERROR_INVALID_VALUE
    assert cb(k=0) == mxg.ERROR_INVALID_VALUE
    assert cb(T=-1) == mxg.ERROR_INVALID_VALUE
    assert cb(ntok=-1) == mxg.ERROR_INVALID_VALUE
    assert cb(out=FAKE_ODD) == mxg.ERROR_INVALID_VALUE
    assert cb(H=12) == mxg.ERROR_NOT_SUPPORTED
    assert cb(ntok=0) == mxg.SUCCESS


def mm(fmt=0, a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, c=FAKE, off=FAKE, ids=FAKE, G=1, E=1, T=4, N=32, K=64):
    return mxg.lib().mx_grouped_matmul(fmt, a, sa, b, sb, c, off, ids, G, E, T, N, K, 0, None)


def test_matmul_argument_errors():
    for kw in [dict(a=None), dict(sa=None), dict(b=None), dict(sb=None), dict(c=None), dict(off=None),
               dict(ids=None), dict(fmt=7), dict(K=0), dict(N=0), dict(E=0), dict(T=-1), dict(G=-1),
               dict(a=FAKE_ODD), dict(c=FAKE_ODD)]:
        assert mm(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert mm(K=40) == mxg.ERROR_NOT_SUPPORTED
    assert mm(G=2000) == mxg.ERROR_NOT_SUPPORTED
    assert mm(T=0) == mxg.SUCCESS


def sw(fmt=2, a=FAKE, sa=FAKE, w=FAKE, sw_=FAKE, yq=FAKE, ys=FAKE, off=FAKE, ids=FAKE, G=1, E=1, T=4, I=64, K=64):
    return mxg.lib().mx_grouped_matmul_swiglu(fmt, a, sa, w, sw_, yq, ys, off, ids, G, E, T, I, K, 0, None)


def test_swiglu_argument_errors():
    for kw in [dict(a=None), dict(yq=None), dict(ys=None), dict(I=0), dict(fmt=9), dict(yq=FAKE_ODD)]:
        assert sw(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert sw(fmt=0) == mxg.ERROR_NOT_SUPPORTED
    assert sw(I=48) == mxg.ERROR_NOT_SUPPORTED
    assert sw(K=16) == mxg.ERROR_NOT_SUPPORTED
    assert sw(T=0) == mxg.SUCCESS


FAKE_4 = P(0x10004)  # on 4 bytes, not on 16


def test_mx_scale_tensors_must_be_16_byte_aligned():
    """MX block-scale tensors are streamed in 16-byte pieces: a scale pointer
    off 16 bytes is refused by every MX GEMM entry point (every call here is
    refused before a launch)."""
    for fmt in (1, 2):
        assert mm(fmt=fmt, sa=FAKE_4) == mxg.ERROR_INVALID_VALUE
        assert mm(fmt=fmt, sb=FAKE_4) == mxg.ERROR_INVALID_VALUE
    assert sw(sa=FAKE_4) == mxg.ERROR_INVALID_VALUE
    assert sw(sw_=FAKE_4) == mxg.ERROR_INVALID_VALUE
    L = mxg.lib()
    for sa, sb in ((FAKE_4, FAKE), (FAKE, FAKE_4)):
        assert L.mx_grouped_matmul_padded(2, FAKE, sa, FAKE, 8, FAKE, sb, FAKE, FAKE, FAKE, 1, 1, 4, 32, 64, 0,
                                          None) == mxg.ERROR_INVALID_VALUE
    assert mm(fmt=0, sa=FAKE_ODD) == mxg.ERROR_INVALID_VALUE  # rowwise fp32 scales: 4 bytes


def test_silu_quantize_argument_errors():
    f = mxg.lib().mx_silu_quantize
    assert f(None, FAKE, FAKE, FAKE, 1, 4, 64, None) == mxg.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 4, 0, None) == mxg.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 4, 40, None) == mxg.ERROR_NOT_SUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 0, 64, None) == mxg.SUCCESS


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mxg.quantize(0, x, torch.tensor([0, 4], dtype=torch.int32))


# Every call below fails validation (or is a no-op with no rows / no groups):
# the fake pointers are never handed to a kernel.
def nq(x=FAKE, qq=FAKE, s=FAKE, sf=FAKE, off=FAKE, ids=FAKE, G=1, E=2, T=4, K=64):
    return mxg.lib().mx_grouped_quantize_nvfp4(x, qq, s, sf, off, ids, G, E, T, K, None)


def test_quantize_nvfp4_argument_errors():
    for kw in [dict(x=None), dict(qq=None), dict(s=None), dict(sf=None), dict(off=None), dict(ids=None), dict(E=0),
               dict(K=0), dict(T=-1), dict(G=-1), dict(x=FAKE_ODD), dict(sf=FAKE_ODD)]:
        assert nq(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert nq(K=24) == mxg.ERROR_NOT_SUPPORTED
    assert nq(G=1025) == mxg.ERROR_NOT_SUPPORTED
    assert nq(T=0) == mxg.SUCCESS
    assert nq(G=0) == mxg.SUCCESS


def nm(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, es=FAKE, c=FAKE, off=FAKE, ids=FAKE, G=1, E=1, T=4, N=32, K=512):
    return mxg.lib().mx_grouped_matmul_nvfp4(a, sa, b, sb, es, c, off, ids, G, E, T, N, K, 0, None)


def test_matmul_nvfp4_argument_errors():
    for kw in [dict(a=None), dict(sa=None), dict(b=None), dict(sb=None), dict(es=None), dict(c=None),
               dict(off=None), dict(ids=None), dict(K=0), dict(N=0), dict(E=0), dict(T=-1), dict(G=-1),
               dict(a=FAKE_ODD), dict(sa=FAKE_ODD), dict(es=FAKE_ODD), dict(c=FAKE_ODD)]:
        assert nm(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert nm(K=256) == mxg.ERROR_NOT_SUPPORTED
    assert nm(G=2000) == mxg.ERROR_NOT_SUPPORTED
    assert nm(T=0) == mxg.SUCCESS


def ns(a=FAKE, sa=FAKE, w=FAKE, ws=FAKE, es=FAKE, rs=None, ysf=FAKE, yq=FAKE, ys=FAKE, off=FAKE, ids=FAKE, G=1, E=1,
       T=4, I=64, K=512):
    return mxg.lib().mx_grouped_matmul_swiglu_nvfp4(a, sa, w, ws, es, rs, ysf, yq, ys, off, ids, G, E, T, I, K, 0,
                                                    None)


def test_swiglu_nvfp4_argument_errors():
    for kw in [dict(a=None), dict(es=None), dict(ysf=None), dict(yq=None), dict(ys=None), dict(I=0), dict(E=0),
               dict(rs=FAKE_ODD), dict(yq=FAKE_ODD), dict(ysf=FAKE_ODD)]:
        assert ns(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert ns(I=48) == mxg.ERROR_NOT_SUPPORTED
    assert ns(K=1000) == mxg.ERROR_NOT_SUPPORTED
    assert ns(T=0) == mxg.SUCCESS


def nsq(h=FAKE, yq=FAKE, ys=FAKE, ysf=FAKE, off=FAKE, ids=FAKE, G=1, E=1, T=4, I=64):
    return mxg.lib().mx_silu_quantize_nvfp4(h, yq, ys, ysf, off, ids, G, E, T, I, None)


def test_silu_quantize_nvfp4_argument_errors():
    for kw in [dict(h=None), dict(yq=None), dict(ys=None), dict(ysf=None), dict(off=None), dict(ids=None),
               dict(I=0), dict(E=0), dict(h=FAKE_ODD)]:
        assert nsq(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert nsq(I=24) == mxg.ERROR_NOT_SUPPORTED
    assert nsq(T=0) == mxg.SUCCESS


def qp(fmt=2, x=FAKE, qq=FAKE, s=FAKE, soff=FAKE, S=16, off=FAKE, G=1, T=4, K=64):
    return mxg.lib().mx_grouped_quantize_padded(fmt, x, qq, s, soff, S, off, G, T, K, None)


def mp(fmt=2, a=FAKE, sa=FAKE, asoff=FAKE, S=16, b=FAKE, sb=FAKE, c=FAKE, off=FAKE, ids=FAKE, G=1, E=1, T=4, N=32,
       K=64):
    return mxg.lib().mx_grouped_matmul_padded(fmt, a, sa, asoff, S, b, sb, c, off, ids, G, E, T, N, K, 0, None)


def sp(fmt=2, a=FAKE, sa=FAKE, asoff=FAKE, S=16, w=FAKE, ws=FAKE, yq=FAKE, ys=FAKE, off=FAKE, ids=FAKE, G=1, E=1,
       T=4, I=64, K=64):
    return mxg.lib().mx_grouped_matmul_swiglu_padded(fmt, a, sa, asoff, S, w, ws, yq, ys, off, ids, G, E, T, I, K, 0,
                                                     None)


def test_padded_argument_errors():
    for kw in [dict(x=None), dict(soff=None), dict(S=-1), dict(fmt=5), dict(soff=FAKE_ODD)]:
        assert qp(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert qp(fmt=0) == mxg.ERROR_NOT_SUPPORTED
    assert qp(K=48) == mxg.ERROR_NOT_SUPPORTED
    assert qp(T=0) == mxg.SUCCESS
    for kw in [dict(asoff=None), dict(S=-1), dict(sa=FAKE_ODD), dict(c=None), dict(fmt=5), dict(asoff=FAKE_ODD)]:
        assert mp(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert mp(fmt=0) == mxg.ERROR_NOT_SUPPORTED
    assert mp(T=0) == mxg.SUCCESS
    for kw in [dict(asoff=None), dict(S=-1), dict(yq=None), dict(I=0)]:
        assert sp(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert sp(fmt=0) == mxg.ERROR_NOT_SUPPORTED
    assert sp(I=48) == mxg.ERROR_NOT_SUPPORTED
    assert sp(T=0) == mxg.SUCCESS


def test_clock_probe_argument_errors():
    L = mxg.lib()
    assert L.mxg_clock_probe(None, 100, None) == mxg.ERROR_INVALID_VALUE
    assert L.mxg_clock_probe(P(0x10004), 100, None) == mxg.ERROR_INVALID_VALUE  # not on 8 bytes
    assert L.mxg_clock_probe(FAKE, 0, None) == mxg.ERROR_INVALID_VALUE
    assert L.mxg_clock_probe(FAKE, 10_000_001, None) == mxg.ERROR_INVALID_VALUE


def test_routing_check_on_host_arrays():
    """The MXG_VALIDATE rule, on host arrays (no GPU): offsets non-decreasing
    and within total_rows, expert ids inside [0, num_experts) when checked."""
    v = mxg.routing_violation
    assert v([0, 3, 5, 9], [0, 1, 2], 3, 9) is None
    assert v([0, 0, 0, 0], [2, 2, 2], 3, 9) is None            # empty groups, repeated experts
    assert v([0], None, 0, 0) is None                          # no groups
    assert "below" in v([0, 3, 2, 9], [0, 1, 2], 3, 9)
    assert "exceeds total_rows" in v([0, 3, 5, 10], [0, 1, 2], 3, 9)
    assert "exceeds total_rows" in v([11, 11, 11, 11], None, 0, 9)
    assert "expert_ids[1] = 3" in v([0, 3, 5, 9], [0, 3, 2], 3, 9)
    assert "expert_ids[0] = -1" in v([0, 3, 5, 9], [-1, 0, 0], 3, 9)
    assert v([0, 3, 5, 9], [0, 3, 2], 0, 9) is None            # ids not checked without num_experts
    assert mxg.lib().mxg_routing_violation(None, None, 1, 1, 4, None, 0) == -1
    assert mxg.lib().mxg_routing_violation(FAKE, None, -1, 1, 4, None, 0) == -1


def test_quantize_scatter_argument_errors():
    f = mxg.lib().mx_grouped_quantize_scatter

    def sc(fmt=0, x=FAKE, ntok=4, ros=FAKE, top_k=2, qq=FAKE, s=FAKE, off=FAKE, G=1, T=8, K=64):
        return f(fmt, x, ntok, ros, top_k, qq, s, off, None, G, T, K, None)

    for kw in [dict(x=None), dict(ros=None), dict(qq=None), dict(s=None), dict(off=None), dict(fmt=5),
               dict(K=0), dict(T=-1), dict(ntok=-1), dict(top_k=0), dict(G=-1), dict(x=FAKE_ODD),
               dict(ros=FAKE_ODD)]:
        assert sc(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert sc(top_k=65) == mxg.ERROR_NOT_SUPPORTED
    assert sc(K=48) == mxg.ERROR_NOT_SUPPORTED
    assert sc(fmt=0, K=8192 + 32) == mxg.ERROR_NOT_SUPPORTED
    assert sc(G=2000) == mxg.ERROR_NOT_SUPPORTED
    assert sc(ntok=0) == mxg.SUCCESS and sc(T=0) == mxg.SUCCESS and sc(G=0) == mxg.SUCCESS


def test_nvfp4_padded_argument_errors():
    L = mxg.lib()

    def nq(x=FAKE, qq=FAKE, s=FAKE, sf=FAKE, soff=FAKE, S=16, off=FAKE, ids=FAKE, G=1, E=1, T=4, K=64):
        return L.mx_grouped_quantize_nvfp4_padded(x, qq, s, sf, soff, S, off, ids, G, E, T, K, None)

    for kw in [dict(x=None), dict(soff=None), dict(sf=None), dict(ids=None), dict(S=-1), dict(E=0), dict(K=0),
               dict(soff=FAKE_ODD), dict(x=FAKE_ODD)]:
        assert nq(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert nq(K=40) == mxg.ERROR_NOT_SUPPORTED
    assert nq(T=0) == mxg.SUCCESS

    def nm(a=FAKE, sa=FAKE, soff=FAKE, S=16, b=FAKE, sb=FAKE, es=FAKE, c=FAKE, off=FAKE, ids=FAKE, G=1, E=1, T=4,
           N=32, K=512):
        return L.mx_grouped_matmul_nvfp4_padded(a, sa, soff, S, b, sb, es, c, off, ids, G, E, T, N, K, 0, None)

    for kw in [dict(a=None), dict(soff=None), dict(es=None), dict(S=-1), dict(sa=FAKE_4), dict(soff=FAKE_ODD),
               dict(E=0)]:
        assert nm(**kw) == mxg.ERROR_INVALID_VALUE, kw
    assert nm(K=256) == mxg.ERROR_NOT_SUPPORTED
    assert nm(T=0) == mxg.SUCCESS


def test_prepared_weights_size_and_argument_errors():
    L = mxg.lib()
    assert mxg.prepared_weights_bytes(3, 96, 128) == 3 * 256 * 128  # N rounded up to whole 256-row tiles
    assert mxg.prepared_weights_bytes(2, 1536, 4096) == 2 * 1536 * 4096
    assert mxg.prepared_weights_bytes(3, 96, 96) == -1   # K not a multiple of 64
    assert mxg.prepared_weights_bytes(0, 96, 128) == -1
    assert mxg.prepared_weights_bytes((1 << 31) - 1, 1 << 29, 1 << 29) == -1  # the size would not fit in int64
    prep = L.mx_prepare_weights_fp8
    assert prep(None, 3, 96, 128, FAKE, None) == mxg.ERROR_INVALID_VALUE
    assert prep(FAKE, 3, 96, 128, None, None) == mxg.ERROR_INVALID_VALUE
    assert prep(FAKE_ODD, 3, 96, 128, FAKE, None) == mxg.ERROR_INVALID_VALUE
    assert prep(FAKE, 0, 96, 128, FAKE, None) == mxg.ERROR_INVALID_VALUE
    assert prep(FAKE, 3, 96, 96, FAKE, None) == mxg.ERROR_NOT_SUPPORTED
    mm = L.mx_grouped_matmul_prepared
    assert mm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 3, 4, 96, 96, None) == mxg.ERROR_NOT_SUPPORTED
    assert mm(FAKE, FAKE, FAKE_ODD, FAKE, FAKE, FAKE, FAKE, 1, 3, 4, 96, 128, None) == mxg.ERROR_INVALID_VALUE
    assert mm(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 3, 4, 96, 128, None) == mxg.ERROR_INVALID_VALUE
    assert mm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 4, 96, 128, None) == mxg.ERROR_INVALID_VALUE
    # no rows: nothing is read, written or launched
    assert mm(None, None, None, None, None, None, None, 1, 3, 0, 96, 128, None) == mxg.SUCCESS


def test_gemm_k_past_the_limit_is_not_supported():
    """Every grouped GEMM entry point refuses K > MXG_MAX_K (its operand loads
    use 32-bit offsets within a tile) before it reads a pointer."""
    L = mxg.lib()
    K = mxg.MAX_K + 512  # a multiple of 32, 64 and 512: only the limit is broken
    NS = mxg.ERROR_NOT_SUPPORTED
    assert mxg.MAX_K == 1 << 22
    for fmt in (mxg.FP8_ROWWISE, mxg.MXFP8, mxg.MXFP4):
        assert L.mx_grouped_matmul(fmt, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 3, 4, 96, K, 0, None) == NS
    for fmt in (mxg.MXFP8, mxg.MXFP4):
        assert L.mx_grouped_matmul_swiglu(fmt, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 3, 4, 64, K, 0,
                                          None) == NS
    assert L.mx_grouped_matmul_prepared(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 3, 4, 96, K, None) == NS
    assert L.mx_grouped_matmul_nvfp4(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 3, 4, 96, K, 0, None) == NS
    assert L.mx_grouped_matmul_swiglu_nvfp4(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 3, 4,
                                            64, K, 0, None) == NS


def test_fp8_tile_choice(monkeypatch):
    """The FP8 tile rule on the shapes it was measured on (N = 1536, K = 4096;
    256 compute units when no device is visible, as here): 256x384 where its
    persistent rounds, weighted 1.4, are fewer, else 256x256; the decode
    regime's 32-row tile for few rows per group; MXG_FP8_TILE forces the
    256-row tile's width (never 384 with N % 8 != 0); malformed sizes give 0."""
    monkeypatch.delenv("MXG_FP8_TILE", raising=False)
    t = mxg.fp8_tile
    # dense: 8k rows fill fewer compute units with 384 columns
    assert t(1, 8192, 1536, 4096, prepared=True) == 256
    assert t(1, 16384, 1536, 4096, prepared=True) == 384
    assert t(1, 65536, 1536, 4096, prepared=True) == 384
    # Zipf-routed over 128 experts: 8k and 16k rows stay 256 wide, the 64k prefill goes 384
    assert t(128, 8192, 1536, 4096, prepared=True) == 256
    assert t(128, 16384, 1536, 4096, prepared=True) == 256
    assert t(128, 65536, 1536, 4096, prepared=True) == 384
    assert t(128, 65536, 1536, 4096, max_rows_per_group_hint=7408) == 384  # row-major, the bench's hint
    assert t(32, 8192, 1536, 4096, prepared=True) == 384
    # the split-round test shape (N = 768)
    assert t(8, 114688, 768, 256, prepared=True) == 384
    # 384 columns would pad N = 1024 to 1152 (256: no padding)
    assert t(1, 1 << 20, 1024, 4096, prepared=True) == 256
    # few rows per group: the decode tile, unless the hint moves the problem up
    assert t(64, 1024, 2048, 7168) == 32
    assert t(64, 1024, 2048, 7168, max_rows_per_group_hint=1 << 20) in (256, 384)
    # K not a multiple of 64: the 128-byte-stage 256 x 256 tile; prepared weights refuse it
    assert t(1, 65536, 1536, 4000) == 256
    assert t(1, 65536, 1536, 4000, prepared=True) == 0
    # malformed sizes
    for args in [(0, 64, 256, 256), (1, 0, 256, 256), (1, 64, 0, 256), (1, 64, 256, 48),
                 (1, 64, 256, mxg.MAX_K + 32), (mxg.MAX_GROUPS + 1, 64, 256, 256)]:
        assert t(*args) == 0, args
    # the override
    monkeypatch.setenv("MXG_FP8_TILE", "256x384")
    assert t(1, 8192, 1536, 4096, prepared=True) == 384
    assert t(1, 8192, 1540, 4096, prepared=True) == 256  # N % 8 != 0
    monkeypatch.setenv("MXG_FP8_TILE", "256x256")
    assert t(128, 65536, 1536, 4096, prepared=True) == 256
    monkeypatch.setenv("MXG_FP8_TILE", "something else")
    assert t(128, 65536, 1536, 4096, prepared=True) == 384
