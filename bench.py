#!/usr/bin/env python3
"""Benchmark of the ragged MoE expert path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload 3] [--no-cpu-baseline]
                    [--settle-seconds 0.2]

A step is one pass of the path over the workload's routed batch: the grouped
dynamic quantize of the bf16 activations, then the grouped GEMM (with its
in-kernel tile map), or the fused gate/up GEMM + SwiGLU + requant for the
fused workload.  Inputs are seeded synthetics already resident in HBM; the
weights are quantized once before timing (offline preparation).

Default workload: prefill_fp8_rowwise (8192 tokens x top-8 of 128 experts,
Zipf(1.1), K=4096, N=1536) -- the configuration the FP8 MFMA target is quoted
on.  `value` is GEMM FLOP per step / step time (TFLOP/s).  The roofline object
describes the GEMM kernel from HIP events recorded around each launch inside
the timed region; the CPU baseline times the oracle on a bounded sample.
Prints ONE JSON line.

Before the warm-up steps the GPU runs the step for a fixed wall time (the
clock settle, reported as `clock_settle_s`): after idle the MI355X clock
overshoots and dips for the first ~30 ms of matrix-core load, and a handful
of warm-up steps would time that transient rather than the kernels.  Working sets that the 256 MB last-level cache could hold
(the quantize of the smaller workloads) are rotated over several copies.
The engine clock the timed steps ran at is measured by the library's clock
probe on a side stream (`gpu_clock`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0}
PEAK_HBM_GBS = 8000.0

METRIC = "ragged MoE grouped GEMM TFLOP/s + % FP8/MXFP4 MFMA peak; quantize GB/s"


# Measured on MI355X: after the GPU goes from idle to this load, the clock
# dips for roughly the first 30-40 ms (prefill GEMM 515 us at step 2, 665 us
# at step 6, back to ~505 us by step 40; the quantize likewise 131 -> 142 ->
# 130 us), so the default warm-up runs for longer than that, and a fixed
# clock settle runs before any warm-up.
WARMUP_SECONDS = 0.1
SETTLE_SECONDS = 0.2
# rotate inputs over copies until the rotated working set exceeds this (the
# MI355X last-level cache holds 256 MB)
ROTATE_BYTES = 512 << 20
MAX_COPIES = 32


def settle(step, seconds):
    """Run `step` in batches of 10 for `seconds` of wall time (untimed)."""
    import torch

    if seconds <= 0:
        return 0
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    return n


class ClockProbe:
    """The library's shader-clock probe, run on a stream of its own while the
    timed steps are repeated (untimed) right after the timed region: one wave
    counts engine-clock ticks against the GPU's constant 100 MHz counter,
    which gives the average clock the steps run at.  (Not during the timed
    steps themselves: the probe's wave takes register space on one compute
    unit, which then cannot host a workgroup of the persistent GEMM.)"""

    def __init__(self, enabled=True):
        self.enabled = enabled
        self.out = None
        self.window_us = 0

    def start(self, window_us):
        import torch

        import fp4_grouped_gemm_quantize_amd as mxg
        if not self.enabled:
            return
        self.window_us = int(max(1, min(window_us, 10_000_000)))
        self.out = torch.zeros(2, dtype=torch.int64, device="cuda")
        self.stream = torch.cuda.Stream()  # default priority
        mxg.clock_probe(self.window_us, self.out, stream=self.stream)

    def result(self):
        if self.out is None:
            return {"error": "not measured (--no-clock)"}
        c, r = (int(v) for v in self.out.cpu())
        if r <= 0:
            return {"error": "probe did not run"}
        return {"mhz": round(100.0 * c / r, 1), "window_us": round(r / 100.0, 1),
                "source": "shader-clock probe (s_memtime vs the 100 MHz counter) on a side stream while the "
                          "timed steps were repeated untimed"}


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def stats_ms(values):
    import numpy as np
    v = np.asarray(values, dtype=np.float64)
    return {"mean": round(float(v.mean()), 4), "median": round(float(np.median(v)), 4), "min": round(float(v.min()), 4)}


def warm_up(step, count):
    """Untimed warm-up: `count` steps, or, with count None, batches of 10
    steps until WARMUP_SECONDS of wall time have passed.  Returns the steps run."""
    import torch

    if count is not None:
        for _ in range(count):
            step()
        torch.cuda.synchronize()
        return count
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARMUP_SECONDS:
            return n


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed warm-up steps (default: whole batches of 10 steps until at least "
                        f"{WARMUP_SECONDS:g} s have passed; the JSON line reports the count)")
    p.add_argument("--workload", type=int, default=3, help="1..5 (default: 3, prefill FP8 rowwise)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-clock", action="store_true", help="do not measure the engine clock during the timed steps")
    p.add_argument("--settle-seconds", type=float, default=SETTLE_SECONDS,
                   help="untimed clock settle before the warm-up steps (wall seconds of steps; 0 disables)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="before the workload, run torch.bitwise_not over this many MiB of int32 three times: a "
                        "streaming kernel that reads and writes a known number of bytes, for scaling rocprofv3's "
                        "FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def algorithmic_gemm_bytes(w, counts, K, N, T, fmt):
    """Each operand read once, output written once; experts with no rows are not read."""
    active = int((counts > 0).sum())
    row_bytes = K // 2 if fmt == 2 else K
    if fmt == 0:
        a = T * row_bytes + T * 4
        b = active * N * (row_bytes + 4)
    else:
        a = T * (row_bytes + K // 32)
        b = active * N * (row_bytes + K // 32)
    out = T * (N // 4 + N // 64) if w.swiglu else T * N * 2
    return a + b + out


def code_text(src):
    """Source text without comments and blank or trailing space, so that the
    hash below follows the code only (the sources hold no comment markers
    inside string literals)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(l.rstrip() for l in src.splitlines() if l.strip())


# the sources the grouped GEMM kernel is compiled from (the kernel whose HBM
# traffic the counter summaries record)
GEMM_SOURCES = ("gemm.hip", "gemm_common.h", "mxg_device.h", "mxg_internal.h")


def kernel_sources_sha():
    """Hash of the GEMM kernel's code (comments excluded): the committed
    counter summaries carry the value they were taken with."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_grouped_gemm_quantize_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def counter_traffic(workload_name):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when the kernels changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256") != kernel_sources_sha():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, r, x_gpu, target_s):
    """The oracle, as it stands, on a bounded sample of the same workload:
    rows from a few groups (quantize + GEMM of those rows against their
    experts).  Returns the value in TFLOP/s of GEMM work."""
    import numpy as np

    import oracle
    import workloads as W

    # the four largest groups, so the sample can reach the time budget
    sel = np.sort(np.argsort(-r.counts, kind="stable")[:min(4, int((r.counts > 0).sum()))])
    wt = W.bf16_bits(W.weights(w, device="cuda", experts=list(sel)))
    E_s = len(sel)
    b, sb = oracle.quantize(w.fmt, wt.reshape(E_s * w.N, w.K), np.array([0, E_s * w.N], np.uint32))
    b = b.reshape(E_s, w.N, -1)
    sb = sb.reshape(E_s, w.N) if w.fmt == 0 else sb.reshape(E_s, w.N, w.K // 32)
    del wt

    def run(rows_per_group):
        rows = []
        for e in sel:
            lo = int(r.row_offsets[e])
            n = min(rows_per_group, int(r.counts[e]))
            rows += list(range(lo, lo + n))
        xs = W.bf16_bits(x_gpu[rows])
        counts = [min(rows_per_group, int(r.counts[e])) for e in sel]
        off = np.r_[0, np.cumsum(counts)].astype(np.uint32)
        ids = np.arange(E_s, dtype=np.int32)
        t0 = time.perf_counter()
        a, sa = oracle.quantize(w.fmt, xs, off)
        if w.swiglu:
            oracle.gemm_swiglu_rows(w.fmt, a, sa, b, sb, off, ids, w.N // 2, w.K, np.arange(len(rows)),
                                    want_exact=False)
        else:
            oracle.gemm_rows(w.fmt, a, sa, b, sb, off, ids, w.N, w.K, np.arange(len(rows)), want_exact=False)
        dt = time.perf_counter() - t0
        return len(rows), dt

    n, dt = run(8)
    per_row = dt / max(n, 1)
    rows_per_group = max(8, int(target_s / per_row / E_s))
    n, dt = run(rows_per_group)
    flops = 2.0 * n * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} routed rows (up to {rows_per_group} from each of the {E_s} largest experts) of the same "
                      f"workload: "
                      f"oracle quantize + grouped GEMM, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "the benchmark measures one GPU: the kernels run on one device and there is no multi-GPU path; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import fp4_grouped_gemm_quantize_amd as mxg
    import workloads as W

    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = (args.copy_calibration_mib << 20) // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    w = W.WORKLOADS[args.workload]
    r = W.routing(w)
    T, K, N, fmt = r.total_rows, w.K, w.N, w.fmt

    # ---- inputs resident in HBM; weights prepared once (untimed)
    x = W.activations(w, r, device="cuda")
    wt = W.weights(w, device="cuda")
    b, sb = mxg.quantize_weights(fmt, wt)
    del wt
    # FP8 rowwise weights go into the layout the GEMM's load ring copies as it
    # is (one-time preparation, like the quantize above), where the row-major
    # GEMM would run that ring too: 128+ rows per group by the library's rule
    # (average rows per non-empty group, moved halfway to the largest group);
    # fewer rows per group stream the weights through the 32-row tile.
    groups = max(1, min(len(r.expert_ids), T))
    avg_rows, top_rows = T // groups, int(r.counts.max())
    regime_rows = (avg_rows + top_rows) // 2 if top_rows > avg_rows else avg_rows
    prepared = (fmt == mxg.FP8_ROWWISE and not w.swiglu and regime_rows >= 128 and
                mxg.prepared_weights_bytes(w.E, N, K) > 0)
    if prepared:
        bp = mxg.prepare_weights_fp8(b)
        del b
    torch.cuda.empty_cache()
    off = torch.from_numpy(r.row_offsets.view(np.int32)).cuda()
    ids = torch.from_numpy(r.expert_ids).cuda()
    qcols = K // 2 if fmt == mxg.MXFP4 else K
    # Copies of the activations and of the quantized rows the step cycles
    # through, so that a working set the last-level cache could hold is not
    # served from it on the next step (one copy when it is large enough).
    q_bytes = T * K * 2 + T * qcols + (T * 4 if fmt == 0 else T * (K // 32))
    copies = int(min(MAX_COPIES, max(1, -(-ROTATE_BYTES // max(q_bytes, 1)))))
    xs_rot = [x] + [x.clone() for _ in range(copies - 1)]
    a_rot = [torch.empty((T, qcols), dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sa_rot = [torch.empty((T,), dtype=torch.float32, device="cuda") if fmt == 0 else
              torch.empty((T, K // 32), dtype=torch.uint8, device="cuda") for _ in range(copies)]
    a, sa = a_rot[0], sa_rot[0]
    if w.swiglu:
        yq = torch.empty((T, N // 4), dtype=torch.uint8, device="cuda")
        ys = torch.empty((T, N // 64), dtype=torch.uint8, device="cuda")
    else:
        c = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    hint = int(r.counts.max())

    cur = [0]

    def quant():
        i = cur[0]
        mxg.mx_grouped_quantize(fmt, xs_rot[i], a_rot[i], sa_rot[i], off, ids)

    def gemm():
        i = cur[0]
        if w.swiglu:
            mxg.mx_grouped_matmul_swiglu(fmt, a_rot[i], sa_rot[i], b, sb, yq, ys, off, ids, hint)
        elif prepared:
            mxg.mx_grouped_matmul_prepared(a_rot[i], sa_rot[i], bp, sb, c, off, ids)
        else:
            mxg.mx_grouped_matmul(fmt, a_rot[i], sa_rot[i], b, sb, c, off, ids, hint)

    def step():
        quant()
        gemm()
        cur[0] = (cur[0] + 1) % copies

    settled = settle(step, args.settle_seconds)
    tw = time.perf_counter()
    warmup = warm_up(step, args.warmup)
    tw = time.perf_counter() - tw
    # expected length of the timed region, for the clock probe's window
    step_s = tw / warmup if warmup else (args.settle_seconds / settled if settled else 1e-3)

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        quant()
        ev[s][1].record(stream)
        gemm()
        ev[s][2].record(stream)
        cur[0] = (cur[0] + 1) % copies
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the engine clock under the same load: the steps again, untimed, beside the probe
    clock = ClockProbe(enabled=not args.no_clock)
    clock.start(0.8 * args.steps * step_s * 1e6)
    for s in range(args.steps):
        step()
    torch.cuda.synchronize()

    q_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(args.steps)]
    g_ms = [ev[s][1].elapsed_time(ev[s][2]) for s in range(args.steps)]
    step_ms = wall * 1e3 / args.steps
    flops = 2.0 * T * N * K
    g_bytes = algorithmic_gemm_bytes(w, r.counts, K, N, T, fmt)
    g_avg = float(np.mean(g_ms))
    q_avg = float(np.mean(q_ms))
    peak = PEAK_TFLOPS["fp4" if fmt == 2 else "fp8"]
    g_tflops = flops / (g_avg * 1e-3) / 1e12
    # the GEMM is MFMA-bound when its intensity exceeds the ridge point
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    mfma_bound = flops / g_bytes >= ridge
    traffic = counter_traffic(w.name)
    roof = {"bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(g_tflops if mfma_bound else g_bytes / (g_avg * 1e-3) / 1e9, 2),
            "peak": peak if mfma_bound else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "traffic": traffic}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    out = {
        "metric": METRIC,
        "value": round(flops / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "clock_settle_s": args.settle_seconds,
        "clock_settle_steps": settled,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4_e2m1" if fmt == 2 else "fp8_e4m3",
        "data": "synthetic (seeded; random-init weights N(0,0.02), activations N(0,1))",
        "config": {"workload": w.name, "routed_rows": T, "experts": w.E, "active_experts": int((r.counts > 0).sum()),
                   "tokens": w.tokens or None, "top_k": w.top_k or None, "K": K, "N": N,
                   "format": mxg.FORMATS[fmt], "routing": w.routing,
                   "weights": "prepared (stage-tiled)" if prepared else "row-major",
                   "max_rows_per_expert": hint, "min_rows_per_expert": int(r.counts.min())},
        "kernels": {
            "quantize_ms": round(q_avg, 4), "quantize_GBps": round(q_bytes / (q_avg * 1e-3) / 1e9, 1),
            "quantize_frac_hbm": round(q_bytes / (q_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "gemm_ms": round(g_avg, 4), "gemm_TFLOPs": round(g_tflops, 1),
            "gemm_frac_mfma_peak": round(g_tflops / peak, 4),
            "gemm_GBps_algorithmic": round(g_bytes / (g_avg * 1e-3) / 1e9, 1),
            "gemm_flop": flops, "gemm_algorithmic_bytes": g_bytes, "quantize_bytes": q_bytes,
            "quantize_ms_stats": stats_ms(q_ms), "gemm_ms_stats": stats_ms(g_ms),
            "input_copies": copies,
        },
        "gpu_clock": clock.result(),
        "roofline": roof,
    }
    if r.token_of_row is not None:
        # the gathered form (routed rows read straight from the token rows),
        # timed on its own; algorithmic bytes: token rows once, codes,
        # scales and indices
        xs = W.source_activations(w, r, device="cuda")
        idx = torch.from_numpy(W.slot_indices(r, w.top_k)).cuda()

        def quant_gather():
            mxg.mx_grouped_quantize_gather(fmt, xs, idx, w.top_k, a, sa, off, ids)

        warm_up(quant_gather, args.warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            quant_gather()
        e1.record(stream)
        torch.cuda.synchronize()
        qg_avg = e0.elapsed_time(e1) / args.steps
        qg_bytes = xs.numel() * 2 + a.numel() + sa.numel() * sa.element_size() + idx.numel() * 4
        out["kernels"].update({"quantize_gather_ms": round(qg_avg, 4),
                               "quantize_gather_GBps": round(qg_bytes / (qg_avg * 1e-3) / 1e9, 1),
                               "quantize_gather_bytes": qg_bytes})
        # the token-major form: each token row read once, stored to its routed rows
        # through the inverse slot map; algorithmic bytes: token rows once,
        # codes, scales and the slot map
        ros = torch.from_numpy(W.rows_of_slots(r, w.top_k, xs.shape[0])).cuda()

        def quant_scatter():
            mxg.mx_grouped_quantize_scatter(fmt, xs, ros, a, sa, off, ids)

        warm_up(quant_scatter, args.warmup)
        e0.record(stream)
        for _ in range(args.steps):
            quant_scatter()
        e1.record(stream)
        torch.cuda.synchronize()
        qs_avg = e0.elapsed_time(e1) / args.steps
        qs_bytes = xs.numel() * 2 + a.numel() + sa.numel() * sa.element_size() + ros.numel() * 4
        out["kernels"].update({"quantize_scatter_ms": round(qs_avg, 4),
                               "quantize_scatter_GBps": round(qs_bytes / (qs_avg * 1e-3) / 1e9, 1),
                               "quantize_scatter_frac_hbm": round(qs_bytes / (qs_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                               "quantize_scatter_bytes": qs_bytes})
        del xs, idx, ros
    if w.swiglu and r.token_of_row is not None:
        # the rest of the expert FFN, timed on its own: the down-projection
        # (MX grouped GEMM with K = I on the fused output, weights [E, H, I])
        # and the combine of each token's top-k rows with router weights
        H, I = K, N // 2
        wd = w.scaled(N=H, K=I, seed=w.seed + 17)
        wdt = W.weights(wd, device="cuda")
        bd, sbd = mxg.quantize_weights(fmt, wdt)
        del wdt
        torch.cuda.empty_cache()
        yd = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        ros = torch.from_numpy(W.rows_of_slots(r, w.top_k, w.tokens)).cuda()
        wts = torch.from_numpy(W.router_weights(w, w.tokens)).cuda()
        comb = torch.empty((w.tokens, H), dtype=torch.bfloat16, device="cuda")

        def down():
            mxg.mx_grouped_matmul(fmt, yq, ys, bd, sbd, yd, off, ids, hint)

        def combine():
            mxg.mx_moe_combine(yd, ros, wts, comb)

        warm_up(lambda: (down(), combine()), args.warmup)
        ed = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        d_ms, c_ms = [], []
        for _ in range(args.steps):
            ed[0].record(stream)
            down()
            ed[1].record(stream)
            combine()
            ed[2].record(stream)
            torch.cuda.synchronize()
            d_ms.append(ed[0].elapsed_time(ed[1]))
            c_ms.append(ed[1].elapsed_time(ed[2]))
        d_avg, c_avg = float(np.mean(d_ms)), float(np.mean(c_ms))
        d_flops = 2.0 * T * H * I
        c_bytes = yd.numel() * 2 + comb.numel() * 2 + ros.numel() * 8
        out["kernels"].update({"down_proj_ms": round(d_avg, 4), "down_proj_TFLOPs": round(d_flops / (d_avg * 1e-3) / 1e12, 1),
                               "down_proj_flop": d_flops, "combine_ms": round(c_avg, 4),
                               "combine_GBps": round(c_bytes / (c_avg * 1e-3) / 1e9, 1), "combine_bytes": c_bytes})
        del bd, sbd, yd, comb
        torch.cuda.empty_cache()
        # The NVFP4 variant of the gate/up GEMM on the same routing: quantize the
        # routed rows (per-expert tensor scale 448*6 / the expert's amax, an
        # input choice) and the plain NVFP4 grouped GEMM with N = 2I (f16
        # matrix cores; no fused epilogue for this format).
        def group_amax(t2d, offs, n):
            am = torch.ones(n, dtype=torch.float32, device=t2d.device)
            rowmax = t2d.abs().amax(dim=1).float()
            for g in range(n):
                lo, hi = int(offs[g]), int(offs[g + 1])
                if hi > lo:
                    am[g] = rowmax[lo:hi].max().clamp_min(1e-30)
            return am
        E = w.E
        sfa = torch.ones(E, dtype=torch.float32, device="cuda")
        am = group_amax(x, r.row_offsets, len(r.expert_ids))
        for g in range(len(r.expert_ids)):
            sfa[int(r.expert_ids[g])] = 2688.0 / am[g]
        wt = W.weights(w, device="cuda")
        sfw = 2688.0 / wt.reshape(E, -1).abs().amax(dim=1).float().clamp_min(1e-30)
        bn, sbn = mxg.quantize_weights_nvfp4(wt, sfw)
        del wt
        torch.cuda.empty_cache()
        esn = (1.0 / (sfa.double() * sfw.double())).float()
        an = torch.empty((T, K // 2), dtype=torch.uint8, device="cuda")
        san = torch.empty((T, K // 16), dtype=torch.uint8, device="cuda")
        cn = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")

        def nv_quant():
            mxg.mx_grouped_quantize_nvfp4(x, an, san, sfa, off, ids)

        def nv_gemm():
            mxg.mx_grouped_matmul_nvfp4(an, san, bn, sbn, esn, cn, off, ids, hint)

        # fused: SwiGLU + NVFP4 requant of y under a per-expert scale (input choice)
        sfy = torch.full((E,), 400.0, dtype=torch.float32, device="cuda")
        yqn = torch.empty((T, N // 4), dtype=torch.uint8, device="cuda")
        ysn = torch.empty((T, N // 32), dtype=torch.uint8, device="cuda")

        def nv_fused():
            mxg.mx_grouped_matmul_swiglu_nvfp4(an, san, bn, sbn, esn, sfy, yqn, ysn, off, ids, None, hint)

        warm_up(lambda: (nv_quant(), nv_gemm(), nv_fused()), args.warmup)
        ed.append(torch.cuda.Event(enable_timing=True))
        nq_ms, ng_ms, nf_ms = [], [], []
        for _ in range(args.steps):
            ed[0].record(stream)
            nv_quant()
            ed[1].record(stream)
            nv_gemm()
            ed[2].record(stream)
            nv_fused()
            ed[3].record(stream)
            torch.cuda.synchronize()
            nq_ms.append(ed[0].elapsed_time(ed[1]))
            ng_ms.append(ed[1].elapsed_time(ed[2]))
            nf_ms.append(ed[2].elapsed_time(ed[3]))
        nq_avg, ng_avg, nf_avg = float(np.mean(nq_ms)), float(np.mean(ng_ms)), float(np.mean(nf_ms))
        nq_bytes = T * K * 2 + T * (K // 2 + K // 16)
        ng_flops = 2.0 * T * N * K
        out["kernels"].update({"nvfp4_quantize_ms": round(nq_avg, 4),
                               "nvfp4_quantize_GBps": round(nq_bytes / (nq_avg * 1e-3) / 1e9, 1),
                               "nvfp4_gemm_ms": round(ng_avg, 4),
                               "nvfp4_gemm_TFLOPs": round(ng_flops / (ng_avg * 1e-3) / 1e12, 1),
                               "nvfp4_gemm_frac_f16_peak": round(ng_flops / (ng_avg * 1e-3) / 2.5e15, 4),
                               "nvfp4_fused_ms": round(nf_avg, 4),
                               "nvfp4_fused_TFLOPs": round(ng_flops / (nf_avg * 1e-3) / 1e12, 1)})
        del bn, sbn, an, san, cn, yqn, ysn
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, r, x, args.cpu_seconds)
        out["cpu_baseline"].update(cpu_info())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
