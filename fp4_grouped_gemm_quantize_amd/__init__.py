"""Python binding of libmxg.so -- the ragged MoE expert path on one gfx950 GPU.

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: if libmxg.so has not been built, every call raises.

Entry points (same names as the C ABI in include/mxg.h):
    mx_grouped_quantize(fmt, x, q, scales, row_offsets, expert_ids=None)
    mx_grouped_matmul(fmt, a_q, a_scales, b_q, b_scales, c, row_offsets, expert_ids, max_rows_per_group_hint=0)
    mx_grouped_matmul_swiglu(fmt, a_q, a_scales, w_q, w_scales, y_q, y_scales, row_offsets, expert_ids,
                             max_rows_per_group_hint=0)
    mx_silu_quantize(h, y_q, y_scales, row_offsets)
plus allocating conveniences quantize(), grouped_matmul(), grouped_matmul_swiglu(), silu_quantize().
"""
from __future__ import annotations

import ctypes
import os

import torch

FP8_ROWWISE = 0
MXFP8 = 1
MXFP4 = 2
FORMATS = {FP8_ROWWISE: "fp8_e4m3_rowwise", MXFP8: "mxfp8_e4m3", MXFP4: "mxfp4_e2m1"}

SUCCESS, ERROR_INVALID_VALUE, ERROR_NOT_SUPPORTED, ERROR_LAUNCH = 0, 1, 2, 3
MAX_GROUPS = 1024
MAX_K = 1 << 22  # largest K of the grouped GEMMs (MXG_MAX_K)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxg.so")

EXPORTED = ("mx_grouped_quantize", "mx_grouped_quantize_gather", "mx_grouped_quantize_scatter", "mx_grouped_matmul", "mx_grouped_matmul_swiglu",
            "mx_silu_quantize", "mx_moe_combine", "mx_grouped_quantize_nvfp4", "mx_grouped_matmul_nvfp4",
            "mx_grouped_matmul_swiglu_nvfp4", "mx_silu_quantize_nvfp4", "mx_grouped_quantize_padded",
            "mx_grouped_matmul_padded", "mx_grouped_matmul_swiglu_padded",
            "mx_grouped_quantize_nvfp4_padded", "mx_grouped_matmul_nvfp4_padded", "mx_prepared_weights_bytes",
            "mx_prepare_weights_fp8", "mx_grouped_matmul_prepared", "mxg_clock_probe", "mxg_fp8_tile",
            "mxg_validation_message", "mxg_routing_violation", "mxg_status_string")


class MxgError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def lib() -> ctypes.CDLL:
    """Load libmxg.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmxg.so not found at {LIB_PATH}: build it with "
                               "`python -m fp4_grouped_gemm_quantize_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.mx_grouped_quantize.argtypes = [ctypes.c_int, _P, _P, _P, _P, _P, _I32, _I64, _I64, _P]
        L.mx_grouped_quantize_gather.argtypes = [ctypes.c_int, _P, _I64, _P, _I32, _P, _P, _P, _P, _I32, _I64, _I64,
                                                 _P]
        L.mx_grouped_quantize_scatter.argtypes = [ctypes.c_int, _P, _I64, _P, _I32, _P, _P, _P, _P, _I32, _I64,
                                                  _I64, _P]
        L.mx_grouped_matmul.argtypes = [ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _I64,
                                        _I64, _P]
        L.mx_grouped_matmul_swiglu.argtypes = [ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64,
                                               _I64, _I64, _I64, _P]
        L.mx_silu_quantize.argtypes = [_P, _P, _P, _P, _I32, _I64, _I64, _P]
        L.mx_moe_combine.argtypes = [_P, _I64, _I64, _P, _P, _I64, _I32, _P, _P]
        L.mx_grouped_quantize_nvfp4.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _P]
        L.mx_grouped_matmul_nvfp4.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _I64, _I64, _P]
        L.mx_grouped_matmul_swiglu_nvfp4.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64,
                                                     _I64, _I64, _I64, _P]
        L.mx_silu_quantize_nvfp4.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _P]
        L.mx_grouped_quantize_padded.argtypes = [ctypes.c_int, _P, _P, _P, _P, _I64, _P, _I32, _I64, _I64, _P]
        L.mx_grouped_matmul_padded.argtypes = [ctypes.c_int, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _I32, _I32,
                                               _I64, _I64, _I64, _I64, _P]
        L.mx_grouped_matmul_swiglu_padded.argtypes = [ctypes.c_int, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _I32,
                                                      _I32, _I64, _I64, _I64, _I64, _P]
        for name in ("mx_grouped_quantize", "mx_grouped_quantize_gather", "mx_grouped_quantize_scatter", "mx_grouped_matmul",
                     "mx_grouped_matmul_swiglu", "mx_silu_quantize", "mx_moe_combine", "mx_grouped_quantize_nvfp4",
                     "mx_grouped_matmul_nvfp4", "mx_grouped_matmul_swiglu_nvfp4", "mx_silu_quantize_nvfp4",
                     "mx_grouped_quantize_padded", "mx_grouped_matmul_padded", "mx_grouped_matmul_swiglu_padded"):
            getattr(L, name).restype = ctypes.c_int
        L.mx_grouped_quantize_nvfp4_padded.argtypes = [_P, _P, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I64, _I64, _P]
        L.mx_grouped_matmul_nvfp4_padded.argtypes = [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64,
                                                     _I64, _I64, _I64, _P]
        L.mx_grouped_quantize_nvfp4_padded.restype = ctypes.c_int
        L.mx_grouped_matmul_nvfp4_padded.restype = ctypes.c_int
        L.mx_prepared_weights_bytes.argtypes = [_I64, _I64, _I64]
        L.mx_prepared_weights_bytes.restype = ctypes.c_int64
        L.mx_prepare_weights_fp8.argtypes = [_P, _I32, _I64, _I64, _P, _P]
        L.mx_prepare_weights_fp8.restype = ctypes.c_int
        L.mx_grouped_matmul_prepared.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _I64, _P]
        L.mx_grouped_matmul_prepared.restype = ctypes.c_int
        L.mxg_validation_message.argtypes = []
        L.mxg_validation_message.restype = ctypes.c_char_p
        L.mxg_routing_violation.argtypes = [_P, _P, _I32, _I32, _I64, ctypes.c_char_p, _I64]
        L.mxg_routing_violation.restype = ctypes.c_int
        L.mxg_clock_probe.argtypes = [_P, _I64, _P]
        L.mxg_clock_probe.restype = ctypes.c_int
        L.mxg_fp8_tile.argtypes = [_I32, _I64, _I64, _I64, _I64, _I32]
        L.mxg_fp8_tile.restype = ctypes.c_int32
        L.mxg_status_string.argtypes = [ctypes.c_int]
        L.mxg_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mxg_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != SUCCESS:
        raise MxgError(status, what)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _expect(t: torch.Tensor, name: str, dtypes, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")


_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_BF16 = (torch.bfloat16,)
_U32 = (torch.uint32, torch.int32)
_I32T = (torch.int32,)


# ----------------------------------------------------------------------------- entry points
def mx_grouped_quantize(fmt: int, x, q, scales, row_offsets, expert_ids=None) -> None:
    """Grouped quantize of bf16 x [T, K] into q / scales (only covered rows written)."""
    _expect(x, "x", _BF16)
    if x.dim() != 2:
        raise ValueError("x must be [total_rows, K]")
    T, K = x.shape
    dev = x.device
    qcols = K // 2 if fmt == MXFP4 else K
    _expect(q, "q", _U8, (T, qcols), dev)
    if fmt == FP8_ROWWISE:
        _expect(scales, "scales", _F32, (T,), dev)
    else:
        _expect(scales, "scales", _U8, (T, K // 32), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    if expert_ids is not None:
        _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_quantize(fmt, _ptr(x), _ptr(q), _ptr(scales), _ptr(row_offsets), _ptr(expert_ids),
                                     G, T, K, _stream(x)), "mx_grouped_quantize")


def mx_grouped_quantize_gather(fmt: int, x_src, indices, indices_divisor: int, q, scales, row_offsets,
                               expert_ids=None) -> None:
    """Grouped quantize of the routed rows x_src[indices[t] // indices_divisor] (x_src bf16
    [S, K], indices int32 [T]) into q / scales [T, ...]; covered rows with an index that
    names no source row are left untouched."""
    _expect(x_src, "x_src", _BF16)
    if x_src.dim() != 2:
        raise ValueError("x_src must be [num_src_rows, K]")
    S, K = x_src.shape
    dev = x_src.device
    _expect(indices, "indices", _I32T, None, dev)
    if indices.dim() != 1:
        raise ValueError("indices must be [total_rows]")
    T = indices.shape[0]
    qcols = K // 2 if fmt == MXFP4 else K
    _expect(q, "q", _U8, (T, qcols), dev)
    if fmt == FP8_ROWWISE:
        _expect(scales, "scales", _F32, (T,), dev)
    else:
        _expect(scales, "scales", _U8, (T, K // 32), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    if expert_ids is not None:
        _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_quantize_gather(fmt, _ptr(x_src), S, _ptr(indices), int(indices_divisor), _ptr(q),
                                            _ptr(scales), _ptr(row_offsets), _ptr(expert_ids), G, T, K,
                                            _stream(x_src)), "mx_grouped_quantize_gather")


def mx_grouped_quantize_scatter(fmt: int, x_tokens, row_of_slot, q, scales, row_offsets, expert_ids=None) -> None:
    """Token-major grouped quantize: each token row of x_tokens [S, K] bf16 is quantized
    once into every routed row row_of_slot[s*top_k + k] (int32 [S * top_k]) of
    q / scales [T, ...] that lies in [0, T) and is covered by a group."""
    _expect(x_tokens, "x_tokens", _BF16)
    if x_tokens.dim() != 2:
        raise ValueError("x_tokens must be [num_tokens, K]")
    S, K = x_tokens.shape
    dev = x_tokens.device
    _expect(row_of_slot, "row_of_slot", _I32T, None, dev)
    if S == 0 or row_of_slot.dim() != 1 or row_of_slot.numel() % S != 0:
        if S != 0:
            raise ValueError("row_of_slot must hold num_tokens * top_k entries")
    top_k = row_of_slot.numel() // S if S else 1
    if q.dim() != 2:
        raise ValueError("q must be [total_rows, K or K/2]")
    T = q.shape[0]
    qcols = K // 2 if fmt == MXFP4 else K
    _expect(q, "q", _U8, (T, qcols), dev)
    if fmt == FP8_ROWWISE:
        _expect(scales, "scales", _F32, (T,), dev)
    else:
        _expect(scales, "scales", _U8, (T, K // 32), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    if expert_ids is not None:
        _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_quantize_scatter(fmt, _ptr(x_tokens), S, _ptr(row_of_slot), top_k, _ptr(q),
                                             _ptr(scales), _ptr(row_offsets), _ptr(expert_ids), G, T, K,
                                             _stream(x_tokens)), "mx_grouped_quantize_scatter")


def mx_grouped_quantize_nvfp4(x, q, scales, tensor_scales, row_offsets, expert_ids) -> None:
    """NVFP4 grouped quantize of bf16 x [T, K] into q u8 [T, K/2] and E4M3 scales u8
    [T, K/16]; the rows of group g use tensor_scales[expert_ids[g]] (fp32 [E])."""
    _expect(x, "x", _BF16)
    if x.dim() != 2:
        raise ValueError("x must be [total_rows, K]")
    T, K = x.shape
    dev = x.device
    _expect(q, "q", _U8, (T, K // 2), dev)
    _expect(scales, "scales", _U8, (T, K // 16), dev)
    _expect(tensor_scales, "tensor_scales", _F32, None, dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_quantize_nvfp4(_ptr(x), _ptr(q), _ptr(scales), _ptr(tensor_scales), _ptr(row_offsets),
                                           _ptr(expert_ids), G, tensor_scales.numel(), T, K, _stream(x)),
           "mx_grouped_quantize_nvfp4")


def mx_grouped_matmul_nvfp4(a_q, a_scales, b_q, b_scales, expert_scales, c, row_offsets, expert_ids,
                            max_rows_per_group_hint: int = 0) -> None:
    """NVFP4 ragged grouped GEMM into bf16 c [T, N]: a_q [T, K/2], a_scales [T, K/16],
    b_q [E, N, K/2], b_scales [E, N, K/16], expert_scales fp32 [E]."""
    _expect(a_q, "a_q", _U8)
    _expect(b_q, "b_q", _U8)
    dev = a_q.device
    T = a_q.shape[0]
    E, N = b_q.shape[0], b_q.shape[1]
    K = a_q.shape[1] * 2
    _expect(b_q, "b_q", _U8, (E, N, K // 2), dev)
    _expect(a_scales, "a_scales", _U8, (T, K // 16), dev)
    _expect(b_scales, "b_scales", _U8, (E, N, K // 16), dev)
    _expect(expert_scales, "expert_scales", _F32, (E,), dev)
    _expect(c, "c", _BF16, (T, N), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_matmul_nvfp4(_ptr(a_q), _ptr(a_scales), _ptr(b_q), _ptr(b_scales), _ptr(expert_scales),
                                         _ptr(c), _ptr(row_offsets), _ptr(expert_ids), G, E, T, N, K,
                                         int(max_rows_per_group_hint), _stream(a_q)), "mx_grouped_matmul_nvfp4")


def mx_grouped_matmul_swiglu_nvfp4(a_q, a_scales, w_q, w_scales, expert_scales, y_tensor_scales, y_q, y_scales,
                                   row_offsets, expert_ids, a_row_scales=None, max_rows_per_group_hint: int = 0) -> None:
    """Fused NVFP4 gate/up grouped GEMM + SwiGLU + NVFP4 requant into y_q [T, I/2],
    y_scales [T, I/16]; y_tensor_scales fp32 [E] (encode side), a_row_scales bf16 [T] or None."""
    _expect(a_q, "a_q", _U8)
    _expect(w_q, "w_q", _U8)
    dev = a_q.device
    T = a_q.shape[0]
    E, N2 = w_q.shape[0], w_q.shape[1]
    I = N2 // 2
    K = a_q.shape[1] * 2
    _expect(w_q, "w_q", _U8, (E, N2, K // 2), dev)
    _expect(a_scales, "a_scales", _U8, (T, K // 16), dev)
    _expect(w_scales, "w_scales", _U8, (E, N2, K // 16), dev)
    _expect(expert_scales, "expert_scales", _F32, (E,), dev)
    _expect(y_tensor_scales, "y_tensor_scales", _F32, (E,), dev)
    if a_row_scales is not None:
        _expect(a_row_scales, "a_row_scales", _BF16, (T,), dev)
    _expect(y_q, "y_q", _U8, (T, I // 2), dev)
    _expect(y_scales, "y_scales", _U8, (T, I // 16), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_matmul_swiglu_nvfp4(_ptr(a_q), _ptr(a_scales), _ptr(w_q), _ptr(w_scales),
                                                _ptr(expert_scales), _ptr(a_row_scales), _ptr(y_tensor_scales),
                                                _ptr(y_q), _ptr(y_scales), _ptr(row_offsets), _ptr(expert_ids), G, E,
                                                T, I, K, int(max_rows_per_group_hint), _stream(a_q)),
           "mx_grouped_matmul_swiglu_nvfp4")


def mx_silu_quantize_nvfp4(h, y_q, y_scales, y_tensor_scales, row_offsets, expert_ids) -> None:
    """SwiGLU + NVFP4 requant of bf16 h [T, 2I] into y_q [T, I/2], y_scales [T, I/16]."""
    _expect(h, "h", _BF16)
    T, N2 = h.shape
    I = N2 // 2
    dev = h.device
    _expect(y_q, "y_q", _U8, (T, I // 2), dev)
    _expect(y_scales, "y_scales", _U8, (T, I // 16), dev)
    _expect(y_tensor_scales, "y_tensor_scales", _F32, None, dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_silu_quantize_nvfp4(_ptr(h), _ptr(y_q), _ptr(y_scales), _ptr(y_tensor_scales), _ptr(row_offsets),
                                        _ptr(expert_ids), G, y_tensor_scales.numel(), T, I, _stream(h)),
           "mx_silu_quantize_nvfp4")


def mx_grouped_quantize_padded(fmt: int, x, q, scales, scales_offsets, row_offsets) -> None:
    """MX grouped quantize of bf16 x [T, K] with group g's scales from row
    scales_offsets[g] of scales [S, K/32] (rows mapped past S are left untouched)."""
    _expect(x, "x", _BF16)
    T, K = x.shape
    dev = x.device
    qcols = K // 2 if fmt == MXFP4 else K
    _expect(q, "q", _U8, (T, qcols), dev)
    _expect(scales, "scales", _U8, None, dev)
    if scales.dim() != 2 or scales.shape[1] != K // 32:
        raise ValueError("scales must be [scale_rows, K/32]")
    _expect(scales_offsets, "scales_offsets", _U32, None, dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    if scales_offsets.numel() < G:
        raise ValueError("scales_offsets needs one entry per group")
    _check(lib().mx_grouped_quantize_padded(fmt, _ptr(x), _ptr(q), _ptr(scales), _ptr(scales_offsets),
                                            scales.shape[0], _ptr(row_offsets), G, T, K, _stream(x)),
           "mx_grouped_quantize_padded")


def mx_grouped_matmul_padded(fmt: int, a_q, a_scales, a_scales_offsets, b_q, b_scales, c, row_offsets, expert_ids,
                             max_rows_per_group_hint: int = 0) -> None:
    """MX grouped GEMM with A's scales [S, K/32] in the padded layout."""
    _expect(a_q, "a_q", _U8)
    dev = a_q.device
    T = a_q.shape[0]
    E, N = b_q.shape[0], b_q.shape[1]
    K = a_q.shape[1] * (2 if fmt == MXFP4 else 1)
    _expect(b_q, "b_q", _U8, (E, N, a_q.shape[1]), dev)
    _expect(a_scales, "a_scales", _U8, None, dev)
    if a_scales.dim() != 2 or a_scales.shape[1] != K // 32:
        raise ValueError("a_scales must be [scale_rows, K/32]")
    _expect(b_scales, "b_scales", _U8, (E, N, K // 32), dev)
    _expect(c, "c", _BF16, (T, N), dev)
    _expect(a_scales_offsets, "a_scales_offsets", _U32, None, dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_matmul_padded(fmt, _ptr(a_q), _ptr(a_scales), _ptr(a_scales_offsets), a_scales.shape[0],
                                          _ptr(b_q), _ptr(b_scales), _ptr(c), _ptr(row_offsets), _ptr(expert_ids), G,
                                          E, T, N, K, int(max_rows_per_group_hint), _stream(a_q)),
           "mx_grouped_matmul_padded")


def mx_grouped_matmul_swiglu_padded(fmt: int, a_q, a_scales, a_scales_offsets, w_q, w_scales, y_q, y_scales,
                                    row_offsets, expert_ids, max_rows_per_group_hint: int = 0) -> None:
    """Fused MX gate/up GEMM + SwiGLU + MXFP4 requant with A's scales in the padded layout."""
    _expect(a_q, "a_q", _U8)
    dev = a_q.device
    T = a_q.shape[0]
    E, N2 = w_q.shape[0], w_q.shape[1]
    I = N2 // 2
    K = a_q.shape[1] * (2 if fmt == MXFP4 else 1)
    _expect(w_q, "w_q", _U8, (E, N2, a_q.shape[1]), dev)
    _expect(a_scales, "a_scales", _U8, None, dev)
    if a_scales.dim() != 2 or a_scales.shape[1] != K // 32:
        raise ValueError("a_scales must be [scale_rows, K/32]")
    _expect(w_scales, "w_scales", _U8, (E, N2, K // 32), dev)
    _expect(y_q, "y_q", _U8, (T, I // 2), dev)
    _expect(y_scales, "y_scales", _U8, (T, I // 32), dev)
    _expect(a_scales_offsets, "a_scales_offsets", _U32, None, dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_matmul_swiglu_padded(fmt, _ptr(a_q), _ptr(a_scales), _ptr(a_scales_offsets),
                                                 a_scales.shape[0], _ptr(w_q), _ptr(w_scales), _ptr(y_q),
                                                 _ptr(y_scales), _ptr(row_offsets), _ptr(expert_ids), G, E, T, I, K,
                                                 int(max_rows_per_group_hint), _stream(a_q)),
           "mx_grouped_matmul_swiglu_padded")


def mx_grouped_matmul(fmt: int, a_q, a_scales, b_q, b_scales, c, row_offsets, expert_ids,
                      max_rows_per_group_hint: int = 0) -> None:
    """Ragged grouped GEMM into bf16 c [T, N] (only covered rows written)."""
    _expect(a_q, "a_q", _U8)
    _expect(b_q, "b_q", _U8)
    dev = a_q.device
    T = a_q.shape[0]
    E, N = b_q.shape[0], b_q.shape[1]
    K = a_q.shape[1] * (2 if fmt == MXFP4 else 1)
    _expect(b_q, "b_q", _U8, (E, N, a_q.shape[1]), dev)
    if fmt == FP8_ROWWISE:
        _expect(a_scales, "a_scales", _F32, (T,), dev)
        _expect(b_scales, "b_scales", _F32, (E, N), dev)
    else:
        _expect(a_scales, "a_scales", _U8, (T, K // 32), dev)
        _expect(b_scales, "b_scales", _U8, (E, N, K // 32), dev)
    _expect(c, "c", _BF16, (T, N), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_matmul(fmt, _ptr(a_q), _ptr(a_scales), _ptr(b_q), _ptr(b_scales), _ptr(c),
                                   _ptr(row_offsets), _ptr(expert_ids), G, E, T, N, K,
                                   int(max_rows_per_group_hint), _stream(a_q)), "mx_grouped_matmul")


def fp8_tile(num_groups: int, total_rows: int, N: int, K: int, max_rows_per_group_hint: int = 0,
             prepared: bool = False) -> int:
    """The tile an FP8 rowwise grouped GEMM of these sizes would run: 384 or 256 (256-row
    tiles of that many columns), 32 (the decode-regime tile), 0 (nothing / refused)."""
    return int(lib().mxg_fp8_tile(int(num_groups), int(total_rows), int(N), int(K),
                                  int(max_rows_per_group_hint), 1 if prepared else 0))


def prepared_weights_bytes(num_experts: int, N: int, K: int) -> int:
    """Bytes of FP8 rowwise weights [E, N, K] in the prepared layout (-1: not preparable)."""
    return int(lib().mx_prepared_weights_bytes(int(num_experts), int(N), int(K)))


def mx_prepare_weights_fp8(b_q, b_prepared) -> None:
    """FP8 rowwise weights b_q u8 [E, N, K] (K a multiple of 64) into b_prepared, a u8
    tensor of prepared_weights_bytes(E, N, K) bytes: the layout the prepared GEMM reads."""
    _expect(b_q, "b_q", _U8)
    if b_q.dim() != 3:
        raise ValueError("b_q must be [num_experts, N, K]")
    E, N, K = b_q.shape
    n = prepared_weights_bytes(E, N, K)
    if n < 0:
        raise ValueError(f"weights [{E}, {N}, {K}] cannot be prepared (K must be a multiple of 64)")
    _expect(b_prepared, "b_prepared", _U8, None, b_q.device)
    if b_prepared.numel() != n or not b_prepared.is_contiguous():
        raise ValueError(f"b_prepared must be a contiguous u8 tensor of {n} bytes")
    _check(lib().mx_prepare_weights_fp8(_ptr(b_q), E, N, K, _ptr(b_prepared), _stream(b_q)),
           "mx_prepare_weights_fp8")


def mx_grouped_matmul_prepared(a_q, a_scales, b_prepared, b_scales, c, row_offsets, expert_ids) -> None:
    """mx_grouped_matmul (FP8 rowwise) with the weights in the prepared layout; E and N
    come from b_scales [E, N], K from a_q [T, K]."""
    _expect(a_q, "a_q", _U8)
    dev = a_q.device
    T, K = a_q.shape
    _expect(b_scales, "b_scales", _F32, None, dev)
    if b_scales.dim() != 2:
        raise ValueError("b_scales must be [num_experts, N]")
    E, N = b_scales.shape
    n = prepared_weights_bytes(E, N, K)
    if n < 0:
        raise ValueError(f"no prepared layout for [{E}, {N}, {K}] (K must be a multiple of 64)")
    _expect(b_prepared, "b_prepared", _U8, None, dev)
    if b_prepared.numel() != n or not b_prepared.is_contiguous():
        raise ValueError(f"b_prepared must be a contiguous u8 tensor of {n} bytes")
    _expect(a_scales, "a_scales", _F32, (T,), dev)
    _expect(c, "c", _BF16, (T, N), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_matmul_prepared(_ptr(a_q), _ptr(a_scales), _ptr(b_prepared), _ptr(b_scales), _ptr(c),
                                            _ptr(row_offsets), _ptr(expert_ids), G, E, T, N, K, _stream(a_q)),
           "mx_grouped_matmul_prepared")


def mx_grouped_matmul_swiglu(fmt: int, a_q, a_scales, w_q, w_scales, y_q, y_scales, row_offsets, expert_ids,
                             max_rows_per_group_hint: int = 0) -> None:
    """Fused gate/up grouped GEMM + SwiGLU + MXFP4 requant into y_q [T, I/2], y_scales [T, I/32]."""
    _expect(a_q, "a_q", _U8)
    _expect(w_q, "w_q", _U8)
    dev = a_q.device
    T = a_q.shape[0]
    E, N2 = w_q.shape[0], w_q.shape[1]
    I = N2 // 2
    K = a_q.shape[1] * (2 if fmt == MXFP4 else 1)
    _expect(w_q, "w_q", _U8, (E, N2, a_q.shape[1]), dev)
    _expect(a_scales, "a_scales", _U8, (T, K // 32), dev)
    _expect(w_scales, "w_scales", _U8, (E, N2, K // 32), dev)
    _expect(y_q, "y_q", _U8, (T, I // 2), dev)
    _expect(y_scales, "y_scales", _U8, (T, I // 32), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _check(lib().mx_grouped_matmul_swiglu(fmt, _ptr(a_q), _ptr(a_scales), _ptr(w_q), _ptr(w_scales), _ptr(y_q),
                                          _ptr(y_scales), _ptr(row_offsets), _ptr(expert_ids), G, E, T, I, K,
                                          int(max_rows_per_group_hint), _stream(a_q)),
           "mx_grouped_matmul_swiglu")


def mx_silu_quantize(h, y_q, y_scales, row_offsets) -> None:
    """SwiGLU + MXFP4 requant of bf16 h [T, 2I] (gate/up interleaved by column)."""
    _expect(h, "h", _BF16)
    dev = h.device
    T, N2 = h.shape
    I = N2 // 2
    _expect(y_q, "y_q", _U8, (T, I // 2), dev)
    _expect(y_scales, "y_scales", _U8, (T, I // 32), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _check(lib().mx_silu_quantize(_ptr(h), _ptr(y_q), _ptr(y_scales), _ptr(row_offsets), G, T, I, _stream(h)),
           "mx_silu_quantize")


def mx_moe_combine(y, row_of_slot, weights, out) -> None:
    """out [tokens, H] bf16 = router-weighted sum over each token's slots of the routed rows
    y [T, H] bf16; row_of_slot int32 / weights fp32 [tokens * top_k] (top_k from out)."""
    _expect(y, "y", _BF16)
    dev = y.device
    T, H = y.shape
    _expect(out, "out", _BF16, None, dev)
    if out.dim() != 2 or out.shape[1] != H:
        raise ValueError("out must be [num_tokens, H]")
    ntok = out.shape[0]
    _expect(row_of_slot, "row_of_slot", _I32T, None, dev)
    _expect(weights, "weights", _F32, None, dev)
    if ntok == 0 or row_of_slot.numel() % ntok != 0 or weights.numel() != row_of_slot.numel():
        if ntok != 0:
            raise ValueError("row_of_slot and weights must hold num_tokens * top_k entries")
    top_k = row_of_slot.numel() // ntok if ntok else 1
    _check(lib().mx_moe_combine(_ptr(y), T, H, _ptr(row_of_slot), _ptr(weights), ntok, top_k, _ptr(out),
                                _stream(y)), "mx_moe_combine")


# ----------------------------------------------------------------------------- allocating forms
def quantize(fmt: int, x, row_offsets, expert_ids=None):
    """Returns (q, scales); rows no group covers are zero."""
    T, K = x.shape
    q = torch.zeros((T, K // 2 if fmt == MXFP4 else K), dtype=torch.uint8, device=x.device)
    if fmt == FP8_ROWWISE:
        s = torch.zeros((T,), dtype=torch.float32, device=x.device)
    else:
        s = torch.zeros((T, K // 32), dtype=torch.uint8, device=x.device)
    mx_grouped_quantize(fmt, x, q, s, row_offsets, expert_ids)
    return q, s


def quantize_gather(fmt: int, x_src, indices, indices_divisor: int, row_offsets, expert_ids=None):
    """Returns (q, scales) for the routed rows x_src[indices // indices_divisor]; rows no
    group covers (or whose index names no source row) are zero."""
    T, K = indices.shape[0], x_src.shape[1]
    q = torch.zeros((T, K // 2 if fmt == MXFP4 else K), dtype=torch.uint8, device=x_src.device)
    if fmt == FP8_ROWWISE:
        s = torch.zeros((T,), dtype=torch.float32, device=x_src.device)
    else:
        s = torch.zeros((T, K // 32), dtype=torch.uint8, device=x_src.device)
    mx_grouped_quantize_gather(fmt, x_src, indices, indices_divisor, q, s, row_offsets, expert_ids)
    return q, s


def grouped_matmul(fmt: int, a_q, a_scales, b_q, b_scales, row_offsets, expert_ids, max_rows_per_group_hint=0):
    c = torch.zeros((a_q.shape[0], b_q.shape[1]), dtype=torch.bfloat16, device=a_q.device)
    mx_grouped_matmul(fmt, a_q, a_scales, b_q, b_scales, c, row_offsets, expert_ids, max_rows_per_group_hint)
    return c


def grouped_matmul_swiglu(fmt: int, a_q, a_scales, w_q, w_scales, row_offsets, expert_ids,
                          max_rows_per_group_hint=0):
    T, I = a_q.shape[0], w_q.shape[1] // 2
    yq = torch.zeros((T, I // 2), dtype=torch.uint8, device=a_q.device)
    ys = torch.zeros((T, I // 32), dtype=torch.uint8, device=a_q.device)
    mx_grouped_matmul_swiglu(fmt, a_q, a_scales, w_q, w_scales, yq, ys, row_offsets, expert_ids,
                             max_rows_per_group_hint)
    return yq, ys


def silu_quantize(h, row_offsets):
    T, I = h.shape[0], h.shape[1] // 2
    yq = torch.zeros((T, I // 2), dtype=torch.uint8, device=h.device)
    ys = torch.zeros((T, I // 32), dtype=torch.uint8, device=h.device)
    mx_silu_quantize(h, yq, ys, row_offsets)
    return yq, ys


def moe_combine(y, row_of_slot, weights, num_tokens: int):
    out = torch.empty((num_tokens, y.shape[1]), dtype=torch.bfloat16, device=y.device)
    mx_moe_combine(y, row_of_slot, weights, out)
    return out


def quantize_weights(fmt: int, w):
    """Quantize bf16 weights [E, N, K] per output row: one group of E*N rows."""
    E, N, K = w.shape
    flat = w.reshape(E * N, K)
    off = torch.tensor([0, E * N], dtype=torch.int32, device=w.device)
    q, s = quantize(fmt, flat, off)
    if fmt == FP8_ROWWISE:
        return q.reshape(E, N, -1), s.reshape(E, N)
    return q.reshape(E, N, -1), s.reshape(E, N, K // 32)


def prepare_weights_fp8(b_q):
    """Allocating form of mx_prepare_weights_fp8: returns the prepared weights (flat u8)."""
    E, N, K = b_q.shape
    n = prepared_weights_bytes(E, N, K)
    if n < 0:
        raise ValueError(f"weights [{E}, {N}, {K}] cannot be prepared (K must be a multiple of 64)")
    out = torch.empty((n,), dtype=torch.uint8, device=b_q.device)
    mx_prepare_weights_fp8(b_q, out)
    return out


def grouped_matmul_prepared(a_q, a_scales, b_prepared, b_scales, row_offsets, expert_ids):
    T = a_q.shape[0]
    c = torch.empty((T, b_scales.shape[1]), dtype=torch.bfloat16, device=a_q.device)
    mx_grouped_matmul_prepared(a_q, a_scales, b_prepared, b_scales, c, row_offsets, expert_ids)
    return c


def quantize_nvfp4(x, row_offsets, expert_ids, tensor_scales):
    T, K = x.shape
    q = torch.zeros((T, K // 2), dtype=torch.uint8, device=x.device)
    s = torch.zeros((T, K // 16), dtype=torch.uint8, device=x.device)
    mx_grouped_quantize_nvfp4(x, q, s, tensor_scales, row_offsets, expert_ids)
    return q, s


def quantize_weights_nvfp4(w, tensor_scales):
    """NVFP4 weights [E, N, K]: one group of N rows per expert under tensor_scales[e]."""
    E, N, K = w.shape
    off = torch.arange(0, (E + 1) * N, N, dtype=torch.int32, device=w.device)
    ids = torch.arange(E, dtype=torch.int32, device=w.device)
    q, s = quantize_nvfp4(w.reshape(E * N, K), off, ids, tensor_scales)
    return q.reshape(E, N, K // 2), s.reshape(E, N, K // 16)


def clock_probe(window_us: int, out: torch.Tensor, stream=None) -> None:
    """Enqueue the shader-clock probe (one wave sleeping window_us of the GPU's
    100 MHz counter) on `stream` (default: the current stream); afterwards
    out[0] / out[1] * 100 MHz is the average engine clock over the window.
    out: int64 [2] on the GPU."""
    _expect(out, "out", (torch.int64,), shape=(2,))
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(out)
    _check(lib().mxg_clock_probe(_ptr(out), int(window_us), s), "mxg_clock_probe")


def validation_message() -> str:
    """Under MXG_VALIDATE: the first routing violation of this thread's last refused call."""
    return lib().mxg_validation_message().decode()


def routing_violation(row_offsets, expert_ids=None, num_experts: int = 0, total_rows: int = 0):
    """The MXG_VALIDATE check on host (numpy) arrays: None if the routing is
    well formed, else a description of the first violation."""
    import numpy as np
    off = np.ascontiguousarray(row_offsets, dtype=np.uint32)
    ids = None if expert_ids is None else np.ascontiguousarray(expert_ids, dtype=np.int32)
    msg = ctypes.create_string_buffer(192)
    rc = lib().mxg_routing_violation(off.ctypes.data, None if ids is None else ids.ctypes.data, off.size - 1,
                                     num_experts, total_rows, msg, len(msg))
    if rc < 0:
        raise ValueError("mxg_routing_violation: invalid arguments")
    return msg.value.decode() if rc else None


def mx_grouped_quantize_nvfp4_padded(x, q, scales, tensor_scales, scales_offsets, row_offsets, expert_ids) -> None:
    """NVFP4 grouped quantize of bf16 x [T, K] into q u8 [T, K/2] with the E4M3 scales of
    group g's row t in row scales_offsets[g] + (t - row_offsets[g]) of scales u8 [S, K/16]."""
    _expect(x, "x", _BF16)
    T, K = x.shape
    dev = x.device
    _expect(q, "q", _U8, (T, K // 2), dev)
    _expect(scales, "scales", _U8, None, dev)
    if scales.dim() != 2 or scales.shape[1] != K // 16:
        raise ValueError("scales must be [scale_rows, K/16]")
    _expect(tensor_scales, "tensor_scales", _F32, None, dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _expect(scales_offsets, "scales_offsets", _U32, (G,), dev)
    _check(lib().mx_grouped_quantize_nvfp4_padded(_ptr(x), _ptr(q), _ptr(scales), _ptr(tensor_scales),
                                                  _ptr(scales_offsets), scales.shape[0], _ptr(row_offsets),
                                                  _ptr(expert_ids), G, tensor_scales.numel(), T, K, _stream(x)),
           "mx_grouped_quantize_nvfp4_padded")


def mx_grouped_matmul_nvfp4_padded(a_q, a_scales, a_scales_offsets, b_q, b_scales, expert_scales, c, row_offsets,
                                   expert_ids, max_rows_per_group_hint: int = 0) -> None:
    """NVFP4 grouped GEMM with A's E4M3 scales in the padded layout (a_scales u8 [S, K/16])."""
    _expect(a_q, "a_q", _U8)
    T, K2 = a_q.shape
    K = 2 * K2
    dev = a_q.device
    _expect(a_scales, "a_scales", _U8, None, dev)
    if a_scales.dim() != 2 or a_scales.shape[1] != K // 16:
        raise ValueError("a_scales must be [scale_rows, K/16]")
    _expect(b_q, "b_q", _U8, None, dev)
    E, N, _ = b_q.shape
    _expect(b_scales, "b_scales", _U8, (E, N, K // 16), dev)
    _expect(expert_scales, "expert_scales", _F32, (E,), dev)
    _expect(c, "c", _BF16, (T, N), dev)
    _expect(row_offsets, "row_offsets", _U32, None, dev)
    G = row_offsets.numel() - 1
    _expect(expert_ids, "expert_ids", _I32T, (G,), dev)
    _expect(a_scales_offsets, "a_scales_offsets", _U32, (G,), dev)
    _check(lib().mx_grouped_matmul_nvfp4_padded(_ptr(a_q), _ptr(a_scales), _ptr(a_scales_offsets), a_scales.shape[0],
                                                _ptr(b_q), _ptr(b_scales), _ptr(expert_scales), _ptr(c),
                                                _ptr(row_offsets), _ptr(expert_ids), G, E, T, N, K,
                                                int(max_rows_per_group_hint), _stream(a_q)),
           "mx_grouped_matmul_nvfp4_padded")
