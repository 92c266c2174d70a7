"""Shared helpers for the parity tests: input preparation (seeded, via
workloads.py), oracle-side preparation, and the comparators.

Inputs always flow from the seeded generators to BOTH sides; the oracle never
receives anything the GPU library produced.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

SENTINEL = 0xA5


def bits(t: torch.Tensor) -> np.ndarray:
    return W.bf16_bits(t)


def to_gpu(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def offsets_gpu(off: np.ndarray) -> torch.Tensor:
    return to_gpu(off.astype(np.uint32).view(np.int32), None).view(torch.int32)


def ids_gpu(ids: np.ndarray) -> torch.Tensor:
    return to_gpu(ids.astype(np.int32))


def sentinel_like(shape, dtype=np.uint8, value=SENTINEL) -> np.ndarray:
    return np.full(shape, value, dtype)


def oracle_quantize_weights(fmt: int, w_bits: np.ndarray):
    """Oracle quantization of bf16 weights [E, N, K] (one group of E*N rows)."""
    E, N, K = w_bits.shape
    off = np.array([0, E * N], np.uint32)
    q, s = oracle.quantize(fmt, w_bits.reshape(E * N, K), off)
    if fmt == oracle.FP8_ROWWISE:
        return q.reshape(E, N, -1), s.reshape(E, N)
    return q.reshape(E, N, -1), s.reshape(E, N, K // 32)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, 2.0 ** (e - 7), 2.0**-133)


def gemm_tolerance(exact: np.ndarray, bound: np.ndarray) -> np.ndarray:
    """|gpu - exact| <= 1e-2 * sum_k |a*b| * scales + one bf16 ulp of the exact value."""
    return 1e-2 * bound + ulp_bf16(exact)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return oracle.bf16_value_array(b)


def sample_rows(off: np.ndarray, rng: np.random.Generator, per_group_extra: int = 0, extra: int = 0):
    """First and last row of every non-empty group, plus random rows."""
    rows = []
    for g in range(off.size - 1):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            rows += [lo, hi - 1]
            if per_group_extra and hi - lo > 2:
                rows += list(rng.integers(lo, hi, per_group_extra))
    T = int(off[-1])
    if extra and T > 0:
        rows += list(rng.integers(0, T, extra))
    return np.unique(np.array(rows, np.int64))


def check_gemm_rows(c_gpu_bits: np.ndarray, ref: dict, label: str = ""):
    """Element-wise tolerance check of gpu rows (bf16 bits [n, N]) against the oracle."""
    g = bf16_bits_to_f64(c_gpu_bits)
    ex = ref["exact"]
    tol = gemm_tolerance(ex, ref["bound"])
    err = np.abs(g - ex)
    ratio = err / tol
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    bad = ~(err <= tol)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} elements outside tolerance; first at ({i},{j}) "
                             f"gpu={g[i, j]!r} exact={ex[i, j]!r} tol={tol[i, j]!r}")
    exact_bf16 = np.mean(c_gpu_bits == ref["out"]) if c_gpu_bits.size else 1.0
    return worst, float(exact_bf16)


# ------------------------------------------------------------------ SwiGLU interval check
_SILU_ARGMIN = -1.2784645427610738  # where silu(z) = z / (1 + e^-z) is smallest


def _silu(z):
    with np.errstate(over="ignore"):  # exp(-z) = inf for very negative z: the limit -0 is right
        return z / (1.0 + np.exp(-z))


def _silu_range(lo, hi):
    a, b = _silu(lo), _silu(hi)
    mn = np.minimum(a, b)
    inside = (lo <= _SILU_ARGMIN) & (_SILU_ARGMIN <= hi)
    mn = np.where(inside, _silu(_SILU_ARGMIN), mn)
    return mn, np.maximum(a, b)


def _e2m1_decode(nib):
    tab = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    return np.where(nib & 8, -tab[nib & 7], tab[nib & 7])


def _floor_log2(a):
    with np.errstate(divide="ignore"):
        return np.floor(np.log2(a))


def check_swiglu_interval(yq_gpu: np.ndarray, ys_gpu: np.ndarray, gu_exact: np.ndarray, gu_bound: np.ndarray):
    """The GPU's fused result must be reachable from SOME gate/up pair inside
    the GEMM tolerance of the exact values: its block scale must arise from an
    amax in the block's interval, and each code must be a rounding of some y
    in the element's interval under that scale.  Returns the fraction of code
    bytes and scale bytes equal to the oracle's own rounding (informational)."""
    tol = gemm_tolerance(gu_exact, gu_bound)
    lo, hi = gu_exact - tol, gu_exact + tol
    # bf16 rounding is monotone: round the interval ends
    lo = oracle.bf16_value_array(oracle.bf16_round_array(lo))
    hi = oracle.bf16_value_array(oracle.bf16_round_array(hi))
    g_lo, g_hi = lo[:, 0::2], hi[:, 0::2]
    u_lo, u_hi = lo[:, 1::2], hi[:, 1::2]
    s_lo, s_hi = _silu_range(g_lo, g_hi)
    corners = np.stack([s_lo * u_lo, s_lo * u_hi, s_hi * u_lo, s_hi * u_hi])
    # widen by the fp32 evaluation error of silu(g) * u (a few ulp of 2^-24)
    c_min, c_max = corners.min(axis=0), corners.max(axis=0)
    c_min = c_min - np.abs(c_min) * 2.0**-20
    c_max = c_max + np.abs(c_max) * 2.0**-20
    y_lo = oracle.bf16_value_array(oracle.bf16_round_array(c_min))
    y_hi = oracle.bf16_value_array(oracle.bf16_round_array(c_max))
    n, I = y_lo.shape
    # block scale interval
    amag_hi = np.maximum(np.abs(y_lo), np.abs(y_hi)).reshape(n, I // 32, 32).max(axis=2)
    amag_lo = np.where((y_lo <= 0) & (y_hi >= 0), 0.0,
                       np.minimum(np.abs(y_lo), np.abs(y_hi))).reshape(n, I // 32, 32).max(axis=2)
    x_lo = np.where(amag_lo > 0, np.clip(_floor_log2(np.maximum(amag_lo, 1e-300)) - 2, -127, 127), -127)
    x_hi = np.where(amag_hi > 0, np.clip(_floor_log2(np.maximum(amag_hi, 1e-300)) - 2, -127, 127), -127)
    X = ys_gpu.astype(np.int64) - 127
    bad_scale = (X < x_lo) | (X > x_hi)
    if bad_scale.any():
        i, b = np.argwhere(bad_scale)[0]
        raise AssertionError(f"scale outside interval at row {i} block {b}: gpu X={X[i, b]} "
                             f"allowed [{x_lo[i, b]}, {x_hi[i, b]}]")
    # element codes under the GPU's own scale
    nib = np.stack([yq_gpu & 0xF, yq_gpu >> 4], axis=-1).reshape(n, I)
    val = _e2m1_decode(nib)
    Xe = np.repeat(X, 32, axis=1).astype(np.float64)
    c_lo = _e2m1_decode(oracle.e2m1_encode_array(y_lo * 2.0 ** (-Xe)))
    c_hi = _e2m1_decode(oracle.e2m1_encode_array(y_hi * 2.0 ** (-Xe)))
    bad = (val < c_lo) | (val > c_hi)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"code outside interval at row {i} output {j}: gpu {val[i, j]} "
                             f"allowed [{c_lo[i, j]}, {c_hi[i, j]}] (y in [{y_lo[i, j]}, {y_hi[i, j]}])")


# ------------------------------------------------------------------ GEMM cases
class GemmCase:
    """Seeded inputs for one grouped GEMM problem, quantized by the ORACLE on the
    CPU; the same code/scale bytes are uploaded for the GPU."""

    def __init__(self, w: W.Workload, gen_device="cpu", routing: "W.Routing | None" = None):
        self.w = w
        self.fmt = w.fmt
        self.r = routing if routing is not None else W.routing(w)
        x = W.activations(w, self.r, device=gen_device)
        wt = W.weights(w, device=gen_device)
        self.x_bits = bits(x)
        del x
        self.a, self.sa = oracle.quantize(self.fmt, self.x_bits, self.r.row_offsets)
        self.b, self.sb = oracle_quantize_weights(self.fmt, bits(wt))
        del wt
        self.off = self.r.row_offsets
        self.ids = self.r.expert_ids
        self.T = int(self.a.shape[0])

    def gpu_inputs(self):
        return dict(a_q=to_gpu(self.a), a_scales=to_gpu(self.sa), b_q=to_gpu(self.b), b_scales=to_gpu(self.sb),
                    row_offsets=offsets_gpu(self.off), expert_ids=ids_gpu(self.ids))

    def oracle_rows(self, rows, N=None):
        N = N if N is not None else self.w.N
        return oracle.gemm_rows(self.fmt, self.a, self.sa, self.b, self.sb, self.off, self.ids, N, self.w.K, rows)


# ---------------------------------------------------------------- guard bytes
GUARD_BYTES = 256
GUARD_PATTERN = 0x5C


class Guarded:
    """A GPU output tensor placed inside a larger allocation with
    GUARD_BYTES of a known pattern before and after it, so a write past
    either end of the tensor is caught (`check()`).  The tensor itself starts
    on a 256-byte boundary, like a fresh allocation, and is contiguous."""

    def __init__(self, init: np.ndarray):
        init = np.ascontiguousarray(init)
        self.nbytes = init.nbytes
        self.buf = torch.full((self.nbytes + 2 * GUARD_BYTES,), GUARD_PATTERN, dtype=torch.uint8, device="cuda")
        inner = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes]
        inner.copy_(torch.from_numpy(init.view(np.uint8).reshape(-1)).cuda())
        self.dtype = init.dtype
        self.shape = init.shape

    def view(self, torch_dtype=None) -> torch.Tensor:
        inner = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes]
        tdt = {np.dtype(np.uint8): torch.uint8, np.dtype(np.int16): torch.int16, np.dtype(np.uint16): torch.int16,
               np.dtype(np.float32): torch.float32, np.dtype(np.int32): torch.int32}[self.dtype]
        t = inner.view(tdt).view(self.shape)
        return t.view(torch_dtype) if torch_dtype is not None else t

    def check(self, label: str = "") -> None:
        head = self.buf[:GUARD_BYTES].cpu().numpy()
        tail = self.buf[GUARD_BYTES + self.nbytes:].cpu().numpy()
        assert np.all(head == GUARD_PATTERN), f"{label}: bytes before the output were written"
        assert np.all(tail == GUARD_PATTERN), f"{label}: bytes after the output were written"

    def numpy(self) -> np.ndarray:
        return self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes].cpu().numpy().view(self.dtype).reshape(self.shape)
