"""bench.py's host-side contract, on the CPU: the one-GPU guard, the default
warm-up rule and the algorithmic byte count the roofline line divides by."""
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    msg = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_default_warm_up_runs_whole_batches_for_the_set_time(monkeypatch):
    import torch

    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    calls = []

    def step():
        calls.append(1)
        time.sleep(0.002)

    t0 = time.perf_counter()
    n = bench.warm_up(step, None)
    assert time.perf_counter() - t0 >= bench.WARMUP_SECONDS
    assert n == len(calls) and n % 10 == 0 and n >= 10
    calls.clear()
    assert bench.warm_up(step, 3) == 3 and len(calls) == 3


def test_prefill_algorithmic_bytes():
    """65,536 routed rows, 128 experts (all active), K = 4096, N = 1536: A codes
    and per-row fp32 scales, each expert's e4m3 weights and per-column fp32
    scales, and the BF16 output, each once."""
    w = W.WORKLOADS[3]
    r = W.routing(w)
    assert r.total_rows == 65536 and int((r.counts > 0).sum()) == 128
    a = 65536 * 4096 + 65536 * 4
    b = 128 * 1536 * 4096 + 128 * 1536 * 4
    c = 65536 * 1536 * 2
    assert bench.algorithmic_gemm_bytes(w, r.counts, w.K, w.N, r.total_rows, w.fmt) == a + b + c == 1276116992


def test_fused_algorithmic_bytes_skip_empty_experts():
    """The MXFP4 fused workload: packed e2m1 codes with E8M0 scales per 32, the
    weights of the experts that receive rows only, and the requantized MXFP4
    output (I/2 code bytes + I/32 scale bytes per row)."""
    w = W.WORKLOADS[5]
    r = W.routing(w)
    active = int((r.counts > 0).sum())
    assert active == w.E - 5
    T, K, I = r.total_rows, w.K, w.N // 2
    a = T * (K // 2 + K // 32)
    b = active * 2 * I * (K // 2 + K // 32)
    y = T * (I // 2 + I // 32)
    assert bench.algorithmic_gemm_bytes(w, np.asarray(r.counts), K, w.N, T, w.fmt) == a + b + y


def test_clock_settle_runs_whole_batches_for_the_set_time(monkeypatch):
    import torch

    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    calls = []

    def step():
        calls.append(1)
        time.sleep(0.001)

    t0 = time.perf_counter()
    n = bench.settle(step, 0.05)
    assert time.perf_counter() - t0 >= 0.05 and n == len(calls) and n % 10 == 0
    assert bench.settle(step, 0) == 0


def test_clock_probe_disabled_reports_why():
    c = bench.ClockProbe(enabled=False)
    c.start(1000)
    assert "error" in c.result()


def test_report_helpers():
    s = bench.stats_ms([1.0, 2.0, 3.0, 10.0])
    assert s == {"mean": 4.0, "median": 2.5, "min": 1.0}
    info = bench.cpu_info()
    assert info["nproc"] >= 1 and info["affinity"] >= 1 and "cpu_model" in info


def test_kernel_hash_follows_code_not_comments():
    a = "int f(int x) {  // the slot\n    /* two\n       lines */ return x + 1;\n}\n"
    b = "int f(int x) {  // another note\n\n    /* changed */ return x + 1;   \n}\n"
    c = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench.code_text(a) == bench.code_text(b) == "int f(int x) {\n     return x + 1;\n}"
    assert bench.code_text(a) != bench.code_text(c)
