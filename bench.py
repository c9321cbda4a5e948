#!/usr/bin/env python3
"""Benchmark of the online-quantized W8A8 linear on one MI355X.

One step = the whole hot path on one batch: online per-token activation
quantization (cider_quant_act) followed by the INT8 MFMA GEMM with the fused
per-channel dequant (cider_w8a8_gemm), at M=4096, N=10240, K=2560 - the
[N=10240, K=2560], M=4096 row of the Cider README's single-op latency table.
Weights are quantized once before timing (the README quantizes them offline).

Prints one JSON line. `value` is whole-step throughput in TOP/s (2*M*N*K
integer ops per step over the step time, quantization included); the
`roofline` object reports the GEMM kernel alone against the MI355X dense INT8
MFMA peak, with its duration taken from HIP events recorded on the stream the
kernels run on; `cpu_baseline` times the CPU oracle on a bounded sample of the
same workload.

Inputs are seeded synthetic tensors (w8a8_online_quantized_amd.inputs): x
~ N(0,1) with 1% outlier channels x20, W ~ N(0, 0.02), fp16. To keep the
weights and activations out of the 256 MB last-level cache between steps the
timed loop rotates over several buffer sets (>= 512 MB in total).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0        # MI355X dense INT8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PAGES_M5PRO_TOPS = 2 * 4096 * 10240 * 2560 / 4.41e-3 / 1e12   # README table: 4.41 ms on Apple M5 Pro
KERNEL_SOURCES = ["cider_api.hip", "cider_quant.hip", "cider_gemm.hip", "cider_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_w8a8_gemm_m4096_n10240_k2560.json")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "w8a8_online_quantized_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(sha: str):
    """HBM bytes per GEMM launch from committed rocprofv3 counter runs, or None
    if they were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != sha:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(M, N, K, budget_s=12.0):
    """The CPU oracle (never tuned) on a bounded row sample of the workload."""
    import numpy as np
    import oracle
    from w8a8_online_quantized_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    w = inputs.weights(N, K, seed=0)
    wq, sw = oracle.quantize_weight(w, 8, 0)
    x = inputs.activations(M, K, seed=0)
    rows_done, chunk = 0, 256
    t0 = time.perf_counter()
    while rows_done < M and time.perf_counter() - t0 < budget_s:
        xs = x[rows_done:rows_done + chunk]
        oracle.w8a8_linear(xs, wq, sw, 0)
        rows_done += xs.shape[0]
    dt = time.perf_counter() - t0
    ops = 2.0 * rows_done * N * K
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows_done} of {M} rows (chunks of {chunk}) of the same M={M},N={N},K={K} "
                      f"per-channel linear: numpy quantize + exact fp64 integer matmul + fp64 dequant, "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--M", type=int, default=4096)
    ap.add_argument("--N", type=int, default=10240)
    ap.add_argument("--K", type=int, default=2560)
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0 = enough for 512 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(collectives and sharding are out of scope); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from w8a8_online_quantized_amd import cider, inputs

    if not torch.cuda.is_available() or not cider.cider_is_available():
        print("bench.py needs a gfx950 GPU and the built libcider.so", file=sys.stderr)
        sys.exit(3)

    M, N, K = args.M, args.N, args.K
    dev = torch.device("cuda:0")
    x_h = torch.from_numpy(inputs.activations(M, K, seed=0))
    w_h = torch.from_numpy(inputs.weights(N, K, seed=0))
    set_bytes = M * K * 2 + M * K + N * K + 2 * M * N + 4 * (M + N)
    R = args.sets or max(2, -(-512 * 2 ** 20 // set_bytes))
    sets = []
    for _ in range(R):
        x = x_h.to(dev)
        wq, sw = cider.cider_quant_weight(w_h.to(dev), 8, 0)
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        sa = torch.empty((M,), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        sets.append((x, xq, sa, wq, sw, y))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(i):
        x, xq, sa, wq, sw, y = sets[i % R]
        cider.cider_quant_act(x, 0, xq, sa, stream=stream)
        cider.cider_w8a8_gemm(xq, sa, wq, sw, 0, y, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        x, xq, sa, wq, sw, y = sets[i % R]
        ev[i][0].record(stream)
        cider.cider_quant_act(x, 0, xq, sa, stream=stream)
        ev[i][1].record(stream)
        cider.cider_w8a8_gemm(xq, sa, wq, sw, 0, y, stream=stream)
        ev[i][2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()

    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    q_ms = [e[0].elapsed_time(e[1]) for e in ev]
    g_ms = [e[1].elapsed_time(e[2]) for e in ev]
    q_avg, g_avg = float(np.mean(q_ms)), float(np.mean(g_ms))
    ops = 2.0 * M * N * K
    value = ops / (ms_step * 1e-3) / 1e12
    gemm_tops = ops / (g_avg * 1e-3) / 1e12
    gemm_bytes = M * K + N * K + 4 * M + 4 * N + 2 * M * N
    quant_bytes = 2 * M * K + M * K + 4 * M

    if args.calib_copy_mb:
        n = args.calib_copy_mb * 2 ** 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    sha = kernel_source_sha()
    out = {
        "metric": "Fused W8A8 GEMM TOPS at M=4096,N=10240,K=2560; % of INT8 MFMA peak",
        "value": round(value, 3),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_M5PRO_TOPS, 3),
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"w8a8 per-channel online-quantized linear, M={M} N={N} K={K}, "
                               f"quant_act + fused GEMM per step",
                   "M": M, "N": N, "K": K, "group_size": 0, "x_dtype": "fp16", "y_dtype": "fp16",
                   "cold_cache_sets": R, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "cider_w8a8_gemm",
                     "achieved": round(gemm_tops, 3), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": measured_traffic(sha),
                     "algorithmic_bytes": gemm_bytes, "algorithmic_ops": ops,
                     "avg_launch_ms": round(g_avg, 5)},
        "kernels": {"cider_quant_act": {"avg_ms": round(q_avg, 5),
                                        "GB/s": round(quant_bytes / (q_avg * 1e-3) / 1e9, 1),
                                        "hbm_frac": round(quant_bytes / (q_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                    "cider_w8a8_gemm": {"avg_ms": round(g_avg, 5), "TOP/s": round(gemm_tops, 2)}},
        "baseline_context": f"Apple M5 Pro, README single-op table: 4.41 ms = {PAGES_M5PRO_TOPS:.1f} TOP/s",
        "kernel_source_sha": sha,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(M, N, K)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
