"""Seeded synthetic inputs for the ragged MoE expert path.

This module only draws random numbers: routings (row offsets, expert ids) and
bf16 activation / weight tensors.  It holds none of the method's arithmetic
(no quantization, no matmul), so both the GPU tests and the CPU oracle can take
their inputs from it.

The five workloads (sizes as named by the project's targets):
  1 tiny_fp8_rowwise     E=4,   128 rows (uniform multinomial), K=256,  N=512
  2 decode_fp8_rowwise   128 tokens x top-8 of 64 experts, K=7168, N=2048,
                         1 % of activation entries scaled x50, 4 experts never
                         routed (so zero-row groups are present)
  3 prefill_fp8_rowwise  8192 tokens x top-8 of 128 experts, Zipf(s=1.1)
                         popularity, K=4096, N=1536
  4 mxfp8                32 experts, 8192 rows split by Dirichlet(0.5), K=7168,
                         N=4096
  5 mxfp4_swiglu         4096 tokens x top-8 of 128 experts, Zipf(s=1.0), 5
                         experts never routed, K=7168, I=2048 (W is [E, 2I, K])

Activations are N(0, 1) and weights N(0, 0.02), drawn in fp32 and rounded to
bf16.  Routed rows of the "tokens x top-k" workloads are copies of their
token's activation row, sorted by (expert, token) as an expert-parallel
dispatch would deliver them; row_offsets is the running count per expert and
expert_ids = 0..E-1, so unrouted experts are zero-length groups.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np
import torch

FP8_ROWWISE = 0
MXFP8 = 1
MXFP4 = 2


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    fmt: int
    E: int
    K: int
    N: int                    # GEMM output width (2I for the fused SwiGLU workload)
    seed: int
    rows: int = 0             # for direct row splits (workloads 1 and 4)
    tokens: int = 0           # for tokens x top-k routings
    top_k: int = 0
    routing: str = "multinomial"  # multinomial | dirichlet | uniform_topk | zipf_topk
    zipf_s: float = 0.0
    alpha: float = 0.0
    masked: int = 0           # experts forced to receive no rows
    outlier_p: float = 0.0
    outlier_mult: float = 1.0
    swiglu: bool = False
    w_std: float = 0.02

    @property
    def I(self) -> int:  # noqa: E743 - the pages' name for the intermediate width
        return self.N // 2

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny_fp8_rowwise", FP8_ROWWISE, E=4, K=256, N=512, seed=101, rows=128,
                routing="multinomial"),
    2: Workload(2, "decode_fp8_rowwise", FP8_ROWWISE, E=64, K=7168, N=2048, seed=102, tokens=128, top_k=8,
                routing="uniform_topk", masked=4, outlier_p=0.01, outlier_mult=50.0),
    3: Workload(3, "prefill_fp8_rowwise", FP8_ROWWISE, E=128, K=4096, N=1536, seed=103, tokens=8192, top_k=8,
                routing="zipf_topk", zipf_s=1.1),
    4: Workload(4, "mxfp8", MXFP8, E=32, K=7168, N=4096, seed=104, rows=8192, routing="dirichlet", alpha=0.5),
    5: Workload(5, "mxfp4_swiglu", MXFP4, E=128, K=7168, N=4096, seed=105, tokens=4096, top_k=8,
                routing="zipf_topk", zipf_s=1.0, masked=5, swiglu=True),
}


@dataclass
class Routing:
    row_offsets: np.ndarray          # uint32 [E+1]
    expert_ids: np.ndarray           # int32 [E]
    token_of_row: np.ndarray | None  # int64 [T] (None when rows are drawn directly)
    counts: np.ndarray = field(default=None)

    @property
    def total_rows(self) -> int:
        return int(self.row_offsets[-1])


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    r, a, b = ss.spawn(3)
    return (np.random.Generator(np.random.PCG64(r)),
            int(a.generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF),
            int(b.generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF))


def _topk_counts(rng, probs: np.ndarray, tokens: int, k: int):
    """Each token picks k distinct experts, Gumbel-top-k on log p."""
    with np.errstate(divide="ignore"):
        logp = np.log(probs)
    choices = np.empty((tokens, k), np.int64)
    for t0 in range(0, tokens, 4096):
        t1 = min(tokens, t0 + 4096)
        gum = rng.gumbel(size=(t1 - t0, probs.size))
        keys = logp[None, :] + gum
        choices[t0:t1] = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return choices


def routing(w: Workload) -> Routing:
    rng, _, _ = _streams(w.seed)
    E = w.E
    token_of_row = None
    if w.routing == "multinomial":
        counts = rng.multinomial(w.rows, np.full(E, 1.0 / E))
    elif w.routing == "dirichlet":
        p = rng.dirichlet(np.full(E, w.alpha))
        counts = rng.multinomial(w.rows, p)
    elif w.routing in ("uniform_topk", "zipf_topk"):
        if w.routing == "uniform_topk":
            p = np.ones(E)
        else:
            ranks = np.arange(1, E + 1, dtype=np.float64)
            p = np.empty(E)
            p[rng.permutation(E)] = ranks ** (-w.zipf_s)
        if w.masked:
            p[rng.choice(E, size=w.masked, replace=False)] = 0.0
        p = p / p.sum()
        choices = _topk_counts(rng, p, w.tokens, w.top_k)
        expert = choices.ravel()
        token = np.repeat(np.arange(w.tokens), w.top_k)
        order = np.lexsort((token, expert))  # by expert, then token
        token_of_row = token[order]
        counts = np.bincount(expert, minlength=E)
    else:
        raise ValueError(w.routing)
    off = np.zeros(E + 1, np.uint32)
    off[1:] = np.cumsum(counts)
    return Routing(off, np.arange(E, dtype=np.int32), token_of_row, counts)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def source_activations(w: Workload, r: Routing, device="cpu") -> torch.Tensor:
    """bf16 source rows, N(0, 1) (with the stated outliers): one per token for
    the tokens x top-k workloads, else one per routed row."""
    _, seed_a, _ = _streams(w.seed)
    g = _gen(device, seed_a)
    n_src = w.tokens if r.token_of_row is not None else r.total_rows
    x = torch.randn((n_src, w.K), generator=g, device=device, dtype=torch.float32)
    if w.outlier_p > 0:
        mask = torch.rand((n_src, w.K), generator=g, device=device) < w.outlier_p
        x = torch.where(mask, x * w.outlier_mult, x)
    return x.to(torch.bfloat16)


def activations(w: Workload, r: Routing, device="cpu") -> torch.Tensor:
    """bf16 [T, K] routed activations: source row token_of_row[t] for row t."""
    x = source_activations(w, r, device)
    if r.token_of_row is not None:
        x = x[torch.as_tensor(r.token_of_row, device=device)]
    return x.contiguous()


def slot_indices(r: Routing, top_k: int) -> np.ndarray:
    """int32 [T] flat slot index token * top_k + k of each routed row, k being
    the row's rank among its token's rows; slot // top_k is the token."""
    tok = np.asarray(r.token_of_row, np.int64)
    seen = np.zeros(int(tok.max()) + 1 if tok.size else 0, np.int64)
    k = np.empty_like(tok)
    for i, t in enumerate(tok):
        k[i] = seen[t]
        seen[t] += 1
    return (tok * top_k + k).astype(np.int32)


def rows_of_slots(r: Routing, top_k: int, num_tokens: int) -> np.ndarray:
    """int32 [num_tokens * top_k]: the routed row of each flat slot (the inverse
    of slot_indices); -1 for a slot no row took."""
    ros = np.full(num_tokens * top_k, -1, np.int32)
    ros[slot_indices(r, top_k)] = np.arange(r.total_rows, dtype=np.int32)
    return ros


def router_weights(w: Workload, num_tokens: int) -> np.ndarray:
    """fp32 [num_tokens * top_k] router weights: a softmax over top_k seeded
    N(0, 1) logits per token (a token's weights sum to about 1)."""
    rng = np.random.default_rng(w.seed + 1000)
    logits = rng.standard_normal((num_tokens, w.top_k))
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32).reshape(-1)


def weights(w: Workload, device="cpu", experts=None) -> torch.Tensor:
    """bf16 [E, N, K] weights, N(0, w_std^2), drawn one expert at a time.

    For the fused SwiGLU workload N = 2I and row 2j of each expert is gate_j,
    row 2j+1 is up_j (the interleaved layout the fused kernel consumes).
    ``experts`` restricts the draw to a subset (same values as the full draw).
    """
    _, _, seed_b = _streams(w.seed)
    ids = range(w.E) if experts is None else experts
    out = torch.empty((len(ids), w.N, w.K), dtype=torch.bfloat16, device=device)
    for i, e in enumerate(ids):
        g = _gen(device, seed_b + 7919 * int(e))
        out[i] = (torch.randn((w.N, w.K), generator=g, device=device, dtype=torch.float32) * w.w_std).to(
            torch.bfloat16)
    return out


def small_variant(w: Workload, **kw) -> Workload:
    """A reduced copy of a workload (same routing law) for oracle-speed tests."""
    return w.scaled(**kw)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw uint16 bit patterns of a bf16 tensor, as a numpy array (CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
