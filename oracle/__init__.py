"""Plain CPU oracle for the ragged MoE expert path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and this package never touches the GPU library: the two share no
code.  The arithmetic lives in ``oracle.c`` (plain C, fp64 where the pages do
not fix a precision); this module only builds it with gcc and marshals numpy
arrays through ctypes.

Pages followed (cited by title and section):
  * grouped_matmul_rowwise_dynamic_scaled_fp8 -- description (the grouped
    formula), Args (shapes and dtypes of c, a, b, a_scales, b_scales,
    a_offsets, expert_ids).
  * grouped_quantize_dynamic_scaled_fp4_async_kernel -- description
    (per-expert BF16 -> MXFP4 / MXFP8 with block scale factors).
  * NvMxf4f8Strategy -- grouped_quantize(), quantize(), grouped_matmul(),
    fused_silu_quantize(), grouped_matmul_swiglu().
  * Struct_ep_dispatch_mxfp4 -- execute (E8M0 activation scales, K_SCALES).
  * NvMxf4f8Strategy -- is_nvfp4, grouped_quantize(input_scale),
    grouped_matmul(expert_scales); the quantize kernel's sf_tensor: NVFP4
    (16-element blocks, E4M3 block scales, per-expert tensor scale; the
    readings are stated in oracle.c).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# Formats, numbered like the GPU library's enum so a test can loop over both.
FP8_ROWWISE = 0
MXFP8 = 1
MXFP4 = 2

_GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU toolchain)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.mxo_num_threads.restype = ctypes.c_int
        for name, res in [("mxo_bf16_value", ctypes.c_double), ("mxo_e4m3_value", ctypes.c_double),
                          ("mxo_e2m1_value", ctypes.c_double), ("mxo_e8m0_value", ctypes.c_double)]:
            fn = getattr(L, name)
            fn.restype = res
        L.mxo_bf16_value.argtypes = [ctypes.c_uint16]
        L.mxo_e4m3_value.argtypes = [ctypes.c_uint8]
        L.mxo_e2m1_value.argtypes = [ctypes.c_uint8]
        L.mxo_e8m0_value.argtypes = [ctypes.c_uint8]
        L.mxo_e4m3_encode.argtypes = [ctypes.c_double]
        L.mxo_e4m3_encode.restype = ctypes.c_uint8
        L.mxo_e2m1_encode.argtypes = [ctypes.c_double]
        L.mxo_e2m1_encode.restype = ctypes.c_uint8
        L.mxo_bf16_round.argtypes = [ctypes.c_double]
        L.mxo_bf16_round.restype = ctypes.c_uint16
        for name in ["mxo_e4m3_encode_array", "mxo_e2m1_encode_array", "mxo_bf16_round_array",
                     "mxo_e4m3_value_array", "mxo_e2m1_value_array"]:
            fn = getattr(L, name)
            fn.argtypes = [_P, _P, _I64]
            fn.restype = None
        L.mxo_group_of_row.argtypes = [_P, _P, _I32, _I32, _I64, _I64]
        L.mxo_group_of_row.restype = _I32
        L.mxo_quantize.argtypes = [ctypes.c_int, _P, _P, _P, _P, _I32, _I64, _I64]
        L.mxo_quantize.restype = ctypes.c_int
        L.mxo_quantize_gather.argtypes = [ctypes.c_int, _P, _I64, _P, _I32, _P, _P, _P, _I32, _I64, _I64]
        L.mxo_quantize_gather.restype = ctypes.c_int
        L.mxo_quantize_scatter.argtypes = [ctypes.c_int, _P, _I64, _P, _I32, _P, _P, _P, _I32, _I64, _I64]
        L.mxo_quantize_scatter.restype = ctypes.c_int
        L.mxo_quantize_nvfp4_padded.argtypes = [_P, _P, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I64, _I64]
        L.mxo_quantize_nvfp4_padded.restype = ctypes.c_int
        L.mxo_combine.argtypes = [_P, _I64, _I64, _P, _P, _I64, _I32, _P, _P, _P]
        L.mxo_combine.restype = ctypes.c_int
        L.mxo_gemm_rows.argtypes = [ctypes.c_int, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _I64,
                                    _P, _I64, _P, _P, _P, _P]
        L.mxo_gemm_rows.restype = ctypes.c_int
        L.mxo_silu_requant.argtypes = [_P, _P, _P, _P, _I32, _I64, _I64, _P]
        L.mxo_silu_requant.restype = ctypes.c_int
        L.mxo_gemm_swiglu_rows.argtypes = [ctypes.c_int, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64,
                                           _I64, _P, _I64, _P, _P, _P, _P, _P]
        L.mxo_gemm_swiglu_rows.restype = ctypes.c_int
        L.mxo_quantize_nvfp4.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64]
        L.mxo_quantize_nvfp4.restype = ctypes.c_int
        L.mxo_gemm_rows_nvfp4.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _I64, _P, _I64,
                                          _P, _P, _P, _P]
        L.mxo_gemm_rows_nvfp4.restype = ctypes.c_int
        L.mxo_silu_requant_nvfp4.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _P]
        L.mxo_silu_requant_nvfp4.restype = ctypes.c_int
        L.mxo_gemm_swiglu_rows_nvfp4.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _I64,
                                                 _P, _I64, _P, _P, _P, _P, _P]
        L.mxo_gemm_swiglu_rows_nvfp4.restype = ctypes.c_int
        L.mxo_quantize_padded.argtypes = [ctypes.c_int, _P, _P, _P, _P, _I64, _P, _I32, _I64, _I64]
        L.mxo_quantize_padded.restype = ctypes.c_int
        L.mxo_gemm_rows_padded.argtypes = [ctypes.c_int, _P, _P, _P, _I64, _P, _P, _P, _P, _I32, _I32, _I64, _I64,
                                           _I64, _P, _I64, _P, _P, _P, _P]
        L.mxo_gemm_rows_padded.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def num_threads() -> int:
    return int(lib().mxo_num_threads())


# ---------------------------------------------------------------- scalar codecs
def bf16_value(bits: int) -> float:
    return lib().mxo_bf16_value(bits)


def e4m3_value(code: int) -> float:
    return lib().mxo_e4m3_value(code)


def e2m1_value(code: int) -> float:
    return lib().mxo_e2m1_value(code)


def e8m0_value(code: int) -> float:
    return lib().mxo_e8m0_value(code)


def e4m3_encode(v: float) -> int:
    return int(lib().mxo_e4m3_encode(float(v)))


def e2m1_encode(v: float) -> int:
    return int(lib().mxo_e2m1_encode(float(v)))


def bf16_round(v: float) -> int:
    return int(lib().mxo_bf16_round(float(v)))


def _map(name, inp, in_dtype, out_dtype):
    x = _c(inp, in_dtype).ravel()
    out = np.empty(x.shape, dtype=out_dtype)
    getattr(lib(), name)(_ptr(x), _ptr(out), x.size)
    return out.reshape(np.shape(inp))


def e4m3_encode_array(v) -> np.ndarray:
    return _map("mxo_e4m3_encode_array", v, np.float64, np.uint8)


def e2m1_encode_array(v) -> np.ndarray:
    return _map("mxo_e2m1_encode_array", v, np.float64, np.uint8)


def bf16_round_array(v) -> np.ndarray:
    return _map("mxo_bf16_round_array", v, np.float64, np.uint16)


def e4m3_value_array(c) -> np.ndarray:
    return _map("mxo_e4m3_value_array", c, np.uint8, np.float64)


def e2m1_value_array(c) -> np.ndarray:
    return _map("mxo_e2m1_value_array", c, np.uint8, np.float64)


def bf16_value_array(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def group_of_row(offsets, expert_ids, num_experts: int, total_rows: int, t: int) -> int:
    off = _c(offsets, np.uint32)
    ids = _c(expert_ids, np.int32) if expert_ids is not None else np.zeros(max(off.size - 1, 1), np.int32)
    return int(lib().mxo_group_of_row(_ptr(off), _ptr(ids), off.size - 1, num_experts, total_rows, t))


# ---------------------------------------------------------------- quantize
def quantize(fmt: int, x_bf16, offsets, q=None, scales=None):
    """Grouped quantize of bf16 bits ``x_bf16`` [T, K] (uint16).

    Returns (q, scales).  Rows not covered by a group keep the contents of the
    passed ``q`` / ``scales`` (zero-filled when not passed).
    fmt 0: q u8 [T, K], scales f32 [T]; fmt 1: q u8 [T, K], scales u8 [T, K/32];
    fmt 2: q u8 [T, K/2] (element 2i in the low nibble), scales u8 [T, K/32].
    """
    x = _c(x_bf16, np.uint16)
    T, K = x.shape
    off = _c(offsets, np.uint32)
    qcols = K // 2 if fmt == MXFP4 else K
    if q is None:
        q = np.zeros((T, qcols), np.uint8)
    if scales is None:
        scales = np.zeros((T,), np.float32) if fmt == FP8_ROWWISE else np.zeros((T, K // 32), np.uint8)
    assert q.shape == (T, qcols) and q.dtype == np.uint8
    rc = lib().mxo_quantize(fmt, _ptr(x), _ptr(q), _ptr(scales), _ptr(off), off.size - 1, T, K)
    if rc != 0:
        raise ValueError("oracle quantize: invalid arguments")
    return q, scales


def quantize_gather(fmt: int, x_src, indices, divisor: int, offsets, q=None, scales=None):
    """Grouped quantize of the routed rows x_src[indices[t] // divisor] (x_src bf16 bits
    [S, K] uint16, indices int32 [T]).  Returns (q, scales) [T, ...]; covered rows whose
    index is negative or names no source row keep their contents, as do uncovered rows."""
    x = _c(x_src, np.uint16)
    S, K = x.shape
    idx = _c(indices, np.int32)
    T = idx.shape[0]
    off = _c(offsets, np.uint32)
    qcols = K // 2 if fmt == MXFP4 else K
    if q is None:
        q = np.zeros((T, qcols), np.uint8)
    if scales is None:
        scales = np.zeros((T,), np.float32) if fmt == FP8_ROWWISE else np.zeros((T, K // 32), np.uint8)
    assert q.shape == (T, qcols) and q.dtype == np.uint8
    rc = lib().mxo_quantize_gather(fmt, _ptr(x), S, _ptr(idx), int(divisor), _ptr(q), _ptr(scales), _ptr(off),
                                   off.size - 1, T, K)
    if rc != 0:
        raise ValueError("oracle quantize_gather: invalid arguments")
    return q, scales


def quantize_scatter(fmt: int, x_tokens, row_of_slot, total_rows: int, offsets, q=None, scales=None):
    """Token-major grouped quantize: token row s (x_tokens bf16 bits [S, K]) is
    quantized once and its result goes to every routed row row_of_slot[s*top_k + k]
    (int32 [S * top_k]) that lies in [0, total_rows) and is covered by a group.
    Returns (q, scales) [total_rows, ...]; every other row keeps its contents."""
    x = _c(x_tokens, np.uint16)
    S, K = x.shape
    ros = _c(row_of_slot, np.int32)
    assert S > 0 and ros.size % S == 0
    top_k = ros.size // S
    T = int(total_rows)
    off = _c(offsets, np.uint32)
    qcols = K // 2 if fmt == MXFP4 else K
    if q is None:
        q = np.zeros((T, qcols), np.uint8)
    if scales is None:
        scales = np.zeros((T,), np.float32) if fmt == FP8_ROWWISE else np.zeros((T, K // 32), np.uint8)
    assert q.shape == (T, qcols) and q.dtype == np.uint8
    rc = lib().mxo_quantize_scatter(fmt, _ptr(x), S, _ptr(ros), top_k, _ptr(q), _ptr(scales), _ptr(off),
                                    off.size - 1, T, K)
    if rc != 0:
        raise ValueError("oracle quantize_scatter: invalid arguments")
    return q, scales


def combine(y_bf16, row_of_slot, weights, num_tokens: int):
    """MoE combine: out[t] = sum_k weights[t*top_k + k] * y[row_of_slot[t*top_k + k]] over
    slots whose row lies in [0, T).  Returns dict with ``out`` (bf16 bits [tokens, H]),
    ``exact`` and ``bound`` (fp64 [tokens, H], bound = sum of |products|)."""
    y = _c(y_bf16, np.uint16)
    T, H = y.shape
    ros = _c(row_of_slot, np.int32)
    w = _c(weights, np.float32)
    assert ros.size == w.size and num_tokens > 0 and ros.size % num_tokens == 0
    top_k = ros.size // num_tokens
    out = np.zeros((num_tokens, H), np.uint16)
    exact = np.zeros((num_tokens, H), np.float64)
    bound = np.zeros((num_tokens, H), np.float64)
    rc = lib().mxo_combine(_ptr(y), T, H, _ptr(ros), _ptr(w), num_tokens, top_k, _ptr(out), _ptr(exact),
                           _ptr(bound))
    if rc != 0:
        raise ValueError("oracle combine: invalid arguments")
    return {"out": out, "exact": exact, "bound": bound}


# ---------------------------------------------------------------- grouped GEMM
def gemm_rows(fmt: int, a, a_scale, b, b_scale, offsets, expert_ids, N: int, K: int, rows,
              want_exact: bool = True):
    """Grouped GEMM output rows ``rows`` (global row indices).

    a: u8 [T, K] (fp8) or [T, K/2] (fp4); b: u8 [E, N, K(/2)].
    Returns dict with ``out`` (bf16 bits [n, N]), ``exact`` and ``bound``
    (fp64 [n, N]) and ``group`` (int32 [n], -1 uncovered, -2 ambiguous).
    """
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    T = a.shape[0]
    E = b.shape[0]
    if fmt == FP8_ROWWISE:
        a_scale = _c(a_scale, np.float32)
        b_scale = _c(b_scale, np.float32)
    else:
        a_scale = _c(a_scale, np.uint8)
        b_scale = _c(b_scale, np.uint8)
    off = _c(offsets, np.uint32)
    ids = _c(expert_ids, np.int32)
    r = _c(rows, np.int64).ravel()
    n = r.size
    out = np.zeros((n, N), np.uint16)
    exact = np.zeros((n, N), np.float64) if want_exact else None
    bound = np.zeros((n, N), np.float64) if want_exact else None
    group = np.zeros((n,), np.int32)
    rc = lib().mxo_gemm_rows(fmt, _ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale), _ptr(off), _ptr(ids),
                             off.size - 1, E, T, N, K, _ptr(r), n, _ptr(out), _ptr(exact), _ptr(bound),
                             _ptr(group))
    if rc != 0:
        raise ValueError("oracle gemm: invalid arguments")
    return {"out": out, "exact": exact, "bound": bound, "group": group}


# ---------------------------------------------------------------- SwiGLU + requant
def silu_requant(h_bf16, offsets, yq=None, ys=None, want_y64: bool = False):
    """Chained gated activation + MXFP4 requant of bf16 [T, 2I] (gate/up interleaved)."""
    h = _c(h_bf16, np.uint16)
    T, N2 = h.shape
    I = N2 // 2
    off = _c(offsets, np.uint32)
    if yq is None:
        yq = np.zeros((T, I // 2), np.uint8)
    if ys is None:
        ys = np.zeros((T, I // 32), np.uint8)
    y64 = np.full((T, I), np.nan, np.float64) if want_y64 else None
    rc = lib().mxo_silu_requant(_ptr(h), _ptr(yq), _ptr(ys), _ptr(off), off.size - 1, T, I, _ptr(y64))
    if rc != 0:
        raise ValueError("oracle silu_requant: invalid arguments")
    return (yq, ys, y64) if want_y64 else (yq, ys)


def gemm_swiglu_rows(fmt: int, a, a_scale, w, w_scale, offsets, expert_ids, I: int, K: int, rows,
                     want_exact: bool = True):
    """Fused gate/up GEMM + SwiGLU + MXFP4 requant for rows ``rows``.

    Returns dict with yq [n, I/2], ys [n, I/32], gu_exact / gu_bound [n, 2I], group [n].
    """
    a = _c(a, np.uint8)
    w = _c(w, np.uint8)
    a_scale = _c(a_scale, np.uint8)
    w_scale = _c(w_scale, np.uint8)
    T = a.shape[0]
    E = w.shape[0]
    off = _c(offsets, np.uint32)
    ids = _c(expert_ids, np.int32)
    r = _c(rows, np.int64).ravel()
    n = r.size
    yq = np.zeros((n, I // 2), np.uint8)
    ys = np.zeros((n, I // 32), np.uint8)
    gu_exact = np.zeros((n, 2 * I), np.float64) if want_exact else None
    gu_bound = np.zeros((n, 2 * I), np.float64) if want_exact else None
    group = np.zeros((n,), np.int32)
    rc = lib().mxo_gemm_swiglu_rows(fmt, _ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(off), _ptr(ids),
                                    off.size - 1, E, T, I, K, _ptr(r), n, _ptr(yq), _ptr(ys), _ptr(gu_exact),
                                    _ptr(gu_bound), _ptr(group))
    if rc != 0:
        raise ValueError("oracle gemm_swiglu: invalid arguments")
    return {"yq": yq, "ys": ys, "gu_exact": gu_exact, "gu_bound": gu_bound, "group": group}


# ---------------------------------------------------------------- NVFP4
NVFP4 = 3


def quantize_nvfp4(x_bf16, offsets, expert_ids, tensor_scales, q=None, scales=None):
    """NVFP4 grouped quantize of bf16 bits ``x_bf16`` [T, K]: rows of group g use
    tensor_scales[expert_ids[g]] (fp32 [E], the encode-side tensor scale).
    Returns (q u8 [T, K/2], scales u8 E4M3 [T, K/16]); uncovered rows keep the
    passed contents (zero-filled when not passed)."""
    x = _c(x_bf16, np.uint16)
    T, K = x.shape
    off = _c(offsets, np.uint32)
    ids = _c(expert_ids, np.int32)
    sf = _c(tensor_scales, np.float32).ravel()
    if q is None:
        q = np.zeros((T, K // 2), np.uint8)
    if scales is None:
        scales = np.zeros((T, K // 16), np.uint8)
    assert q.shape == (T, K // 2) and scales.shape == (T, K // 16)
    rc = lib().mxo_quantize_nvfp4(_ptr(x), _ptr(q), _ptr(scales), _ptr(sf), _ptr(off), _ptr(ids), off.size - 1,
                                  sf.size, T, K)
    if rc != 0:
        raise ValueError("oracle quantize_nvfp4: invalid arguments")
    return q, scales


def gemm_rows_nvfp4(a, a_scale, b, b_scale, expert_scales, offsets, expert_ids, N: int, K: int, rows,
                    want_exact: bool = True):
    """NVFP4 grouped GEMM output rows ``rows``: a u8 [T, K/2], a_scale u8 [T, K/16],
    b u8 [E, N, K/2], b_scale u8 [E, N, K/16], expert_scales fp32 [E].  Same
    return dict as gemm_rows."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    a_scale = _c(a_scale, np.uint8)
    b_scale = _c(b_scale, np.uint8)
    es = _c(expert_scales, np.float32).ravel()
    T = a.shape[0]
    E = b.shape[0]
    off = _c(offsets, np.uint32)
    ids = _c(expert_ids, np.int32)
    r = _c(rows, np.int64).ravel()
    n = r.size
    out = np.zeros((n, N), np.uint16)
    exact = np.zeros((n, N), np.float64) if want_exact else None
    bound = np.zeros((n, N), np.float64) if want_exact else None
    group = np.zeros((n,), np.int32)
    rc = lib().mxo_gemm_rows_nvfp4(_ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale), _ptr(es), _ptr(off), _ptr(ids),
                                   off.size - 1, E, T, N, K, _ptr(r), n, _ptr(out), _ptr(exact), _ptr(bound),
                                   _ptr(group))
    if rc != 0:
        raise ValueError("oracle gemm_nvfp4: invalid arguments")
    return {"out": out, "exact": exact, "bound": bound, "group": group}


def silu_requant_nvfp4(h_bf16, offsets, expert_ids, y_tensor_scales, yq=None, ys=None, want_y64: bool = False):
    """Chained gated activation + NVFP4 requant of bf16 [T, 2I] (gate/up interleaved);
    rows of group g use y_tensor_scales[expert_ids[g]] (encode side).  Returns
    (yq u8 [T, I/2], ys u8 E4M3 [T, I/16]) and, optionally, fp64 y [T, I]."""
    h = _c(h_bf16, np.uint16)
    T, N2 = h.shape
    I = N2 // 2
    off = _c(offsets, np.uint32)
    ids = _c(expert_ids, np.int32)
    sf = _c(y_tensor_scales, np.float32).ravel()
    if yq is None:
        yq = np.zeros((T, I // 2), np.uint8)
    if ys is None:
        ys = np.zeros((T, I // 16), np.uint8)
    y64 = np.full((T, I), np.nan, np.float64) if want_y64 else None
    rc = lib().mxo_silu_requant_nvfp4(_ptr(h), _ptr(yq), _ptr(ys), _ptr(sf), _ptr(off), _ptr(ids), off.size - 1,
                                      sf.size, T, I, _ptr(y64))
    if rc != 0:
        raise ValueError("oracle silu_requant_nvfp4: invalid arguments")
    return (yq, ys, y64) if want_y64 else (yq, ys)


def gemm_swiglu_rows_nvfp4(a, a_scale, w, w_scale, expert_scales, row_scales_bf16, y_tensor_scales, offsets,
                           expert_ids, I: int, K: int, rows, want_exact: bool = True):
    """Fused NVFP4 gate/up GEMM (+ optional bf16 row scales) + SwiGLU + NVFP4 requant
    for ``rows``.  Returns dict with yq [n, I/2], ys [n, I/16], gu_exact / gu_bound
    [n, 2I] and group [n]."""
    a = _c(a, np.uint8)
    w = _c(w, np.uint8)
    a_scale = _c(a_scale, np.uint8)
    w_scale = _c(w_scale, np.uint8)
    es = _c(expert_scales, np.float32).ravel()
    rs = None if row_scales_bf16 is None else _c(row_scales_bf16, np.uint16).ravel()
    sf = _c(y_tensor_scales, np.float32).ravel()
    T = a.shape[0]
    E = w.shape[0]
    off = _c(offsets, np.uint32)
    ids = _c(expert_ids, np.int32)
    r = _c(rows, np.int64).ravel()
    n = r.size
    yq = np.zeros((n, I // 2), np.uint8)
    ys = np.zeros((n, I // 16), np.uint8)
    gu_exact = np.zeros((n, 2 * I), np.float64) if want_exact else None
    gu_bound = np.zeros((n, 2 * I), np.float64) if want_exact else None
    group = np.zeros((n,), np.int32)
    rc = lib().mxo_gemm_swiglu_rows_nvfp4(_ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(es), _ptr(rs),
                                          _ptr(sf), _ptr(off), _ptr(ids), off.size - 1, E, T, I, K, _ptr(r), n,
                                          _ptr(yq), _ptr(ys), _ptr(gu_exact), _ptr(gu_bound), _ptr(group))
    if rc != 0:
        raise ValueError("oracle gemm_swiglu_nvfp4: invalid arguments")
    return {"yq": yq, "ys": ys, "gu_exact": gu_exact, "gu_bound": gu_bound, "group": group}


# ---------------------------------------------------------------- padded MX scale layouts
def quantize_padded(fmt: int, x_bf16, offsets, scales_offsets, scale_rows: int, q=None, scales=None):
    """MX grouped quantize with the scales of group g's row t in row
    scales_offsets[g] + (t - offsets[g]) of a [scale_rows, K/32] tensor; a row whose
    scale row is at or past scale_rows is left untouched.  Returns (q, scales)."""
    x = _c(x_bf16, np.uint16)
    T, K = x.shape
    off = _c(offsets, np.uint32)
    soff = _c(scales_offsets, np.uint32).ravel()
    qcols = K // 2 if fmt == MXFP4 else K
    if q is None:
        q = np.zeros((T, qcols), np.uint8)
    if scales is None:
        scales = np.zeros((scale_rows, K // 32), np.uint8)
    assert soff.size >= off.size - 1 and scales.shape == (scale_rows, K // 32)
    rc = lib().mxo_quantize_padded(fmt, _ptr(x), _ptr(q), _ptr(scales), _ptr(soff), scale_rows, _ptr(off),
                                   off.size - 1, T, K)
    if rc != 0:
        raise ValueError("oracle quantize_padded: invalid arguments")
    return q, scales



def quantize_nvfp4_padded(x_bf16, offsets, expert_ids, tensor_scales, scales_offsets, scale_rows: int, q=None,
                          scales=None):
    """NVFP4 grouped quantize (as quantize_nvfp4) with the E4M3 scales of group g's row t
    in row scales_offsets[g] + (t - offsets[g]) of a [scale_rows, K/16] tensor; a row whose
    scale row is at or past scale_rows is left untouched.  Returns (q, scales)."""
    x = _c(x_bf16, np.uint16)
    T, K = x.shape
    off = _c(offsets, np.uint32)
    ids = _c(expert_ids, np.int32)
    sf = _c(tensor_scales, np.float32)
    soff = _c(scales_offsets, np.uint32).ravel()
    if q is None:
        q = np.zeros((T, K // 2), np.uint8)
    if scales is None:
        scales = np.zeros((scale_rows, K // 16), np.uint8)
    assert soff.size >= off.size - 1 and scales.shape == (scale_rows, K // 16)
    rc = lib().mxo_quantize_nvfp4_padded(_ptr(x), _ptr(q), _ptr(scales), _ptr(sf), _ptr(soff), scale_rows,
                                         _ptr(off), _ptr(ids), off.size - 1, sf.size, T, K)
    if rc != 0:
        raise ValueError("oracle quantize_nvfp4_padded: invalid arguments")
    return q, scales

def gemm_rows_padded(fmt: int, a, a_scale, a_scales_offsets, b, b_scale, offsets, expert_ids, N: int, K: int, rows,
                     want_exact: bool = True):
    """MX grouped GEMM rows with A's scales in a padded layout ([S, K/32], group g's
    rows from row a_scales_offsets[g]); same return dict as gemm_rows."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    a_scale = _c(a_scale, np.uint8)
    b_scale = _c(b_scale, np.uint8)
    asoff = _c(a_scales_offsets, np.uint32).ravel()
    T = a.shape[0]
    E = b.shape[0]
    off = _c(offsets, np.uint32)
    ids = _c(expert_ids, np.int32)
    r = _c(rows, np.int64).ravel()
    n = r.size
    out = np.zeros((n, N), np.uint16)
    exact = np.zeros((n, N), np.float64) if want_exact else None
    bound = np.zeros((n, N), np.float64) if want_exact else None
    group = np.zeros((n,), np.int32)
    rc = lib().mxo_gemm_rows_padded(fmt, _ptr(a), _ptr(a_scale), _ptr(asoff), a_scale.shape[0], _ptr(b),
                                    _ptr(b_scale), _ptr(off), _ptr(ids), off.size - 1, E, T, N, K, _ptr(r), n,
                                    _ptr(out), _ptr(exact), _ptr(bound), _ptr(group))
    if rc != 0:
        raise ValueError("oracle gemm_rows_padded: invalid arguments")
    return {"out": out, "exact": exact, "bound": bound, "group": group}
