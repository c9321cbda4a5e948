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
timed loop rotates over several buffer sets (>= 512 MB in total). The default
100 untimed steps let the GPU reach its sustained clock before the 200 timed
ones (it ramps up over the first ~10 ms of load after idling); before them,
--settle-ms of untimed steps (default 200 ms) let the clock ramp finish even
when few warm-up steps are asked for. No process is spawned once the GPU is
in use: the shader clock is read from sysfs in-process.
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
CSRC = os.path.join(ROOT, "w8a8_online_quantized_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_w8a8_gemm_m4096_n10240_k2560.json")


def kernel_source_sha() -> str:
    """Hash of every source the library is built from (csrc/*.hip, *.h)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
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


def host_cpu_model() -> str:
    """The host CPU's model name, read from /proc/cpuinfo (no process spawned)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_info():
    """(BLAS vendor / library, threads) of numpy's BLAS from threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        if pools:
            p = pools[0]
            name = f"{p.get('internal_api', '?')} {p.get('version', '')}".strip()
            return name, int(max(q.get("num_threads", 1) for q in pools))
    except Exception:  # pragma: no cover
        pass
    return "unknown", os.cpu_count() or 1


def cpu_baseline(M, N, K, budget_s=12.0):
    """The CPU oracle (never tuned) on the same workload for about budget_s
    seconds of host time (whole 256-row chunks, wrapping over the rows)."""
    import numpy as np  # noqa: F401
    import oracle
    from w8a8_online_quantized_amd import inputs
    blas, threads = blas_info()
    w = inputs.weights(N, K, seed=0)
    wq, sw = oracle.quantize_weight(w, 8, 0)
    x = inputs.activations(M, K, seed=0)
    rows_done, chunk = 0, 256
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        start = rows_done % M
        xs = x[start:start + chunk]
        oracle.w8a8_linear(xs, wq, sw, 0)
        rows_done += xs.shape[0]
    dt = time.perf_counter() - t0
    ops = 2.0 * rows_done * N * K
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows_done} rows ({rows_done / M:.2f} passes over the M={M} rows, chunks of {chunk}) "
                      f"of the same N={N}, K={K} per-channel linear: numpy quantize + exact fp64 integer "
                      f"matmul + fp64 dequant, {dt:.1f} s",
            "ms_per_step_equiv": round(dt / (rows_done / M) * 1e3, 2),
            "cpu_model": host_cpu_model(), "os_cpu_count": os.cpu_count(), "blas": blas,
            "blas_threads": int(threads)}


def algorithmic(mode, M, N, K, gs):
    """Integer ops and HBM bytes one GEMM launch must move, and the bytes of the
    activation quantization (fp16 in, int8 + fp32 scales out)."""
    G = 1 if gs == 0 else K // gs
    if mode in ("int8_mv", "w8a8_linear"):   # fp16 x and int8 weights in, fp16 y out, one launch
        return 2.0 * M * N * K, 2 * M * K + N * K + 4 * N * G + 2 * M * N, 0
    wbytes = N * K // 2 if mode == "w4a8" else N * K
    Ga = 1 if mode == "w8a8_tokpg" else G   # per-token activations x per-group weights
    gemm_bytes = M * K + wbytes + 4 * M * Ga + 4 * N * G + 2 * M * N
    quant_bytes = 2 * M * K + M * K + 4 * M * Ga
    return 2.0 * M * N * K, gemm_bytes, quant_bytes


def _sysfs_clock_files():
    """The amdgpu sysfs files that report the current shader clock: the
    DPM table (current level marked '*') and the hwmon frequency input, for
    every card the driver exposes. Read in-process: nothing is spawned."""
    import glob
    dpm = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    hw = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/freq1_input"))
    mem = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_mclk"))
    return dpm, hw, mem


def _read_dpm_mhz(path):
    """MHz of the level marked current ('*') in a pp_dpm_* table, else None."""
    import re
    try:
        with open(path) as f:
            for line in f:
                if "*" in line:
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                    if m:
                        return float(m.group(1))
    except OSError:
        return None
    return None


def _clock_sample(files):
    """(shader clock, memory clock) in MHz now, from sysfs; None if unreadable."""
    dpm, hw, mem = files
    sc = None
    for p in hw:
        try:
            with open(p) as f:
                sc = float(f.read().strip()) / 1e6
            break
        except (OSError, ValueError):
            continue
    if sc is None:
        for p in dpm:
            sc = _read_dpm_mhz(p)
            if sc is not None:
                break
    mc = next((v for v in (_read_dpm_mhz(p) for p in mem) if v is not None), None)
    return (sc, mc) if sc is not None else None


def profiler_attached() -> bool:
    """True under rocprofv3 (its tool library is preloaded / its env is set)."""
    pre = os.environ.get("LD_PRELOAD", "")
    return "rocprof" in pre or any(k.startswith("ROCPROF") for k in os.environ)


def sample_sclk(torch, launch, seconds=1.0):
    """Shader clock (MHz) sampled from sysfs in a helper thread while `launch`
    (one GEMM) runs back to back for `seconds`: (median, min, max, number of
    samples, median memory clock), or None when sysfs reports no clock."""
    import threading
    files = _sysfs_clock_files()
    if not any(files[:2]):
        return None
    samples = []
    stop = time.time() + seconds

    def sampler():
        time.sleep(0.1)
        while time.time() < stop - 0.05:
            v = _clock_sample(files)
            if v:
                samples.append(v)
            time.sleep(0.02)
    t = threading.Thread(target=sampler)
    t.start()
    i = 0
    while time.time() < stop:
        for _ in range(20):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    t.join()
    if not samples:
        return None
    sc = sorted(v[0] for v in samples)
    mc = sorted(v[1] for v in samples if v[1])
    return sc[len(sc) // 2], sc[0], sc[-1], len(sc), (mc[len(mc) // 2] if mc else None)


def measure(cider, torch, inputs, mode, M, N, K, gs, steps, warmup, min_set_bytes=512 * 2 ** 20, clock_s=0.0,
            settle_s=0.0):
    """Times `steps` passes of quant_act + GEMM for one workload, rotating over
    enough buffer sets to keep the working set out of the 256 MB last-level
    cache. Returns the time per step and each kernel's average launch duration,
    all from HIP events on the launch stream (events only around each timed
    loop, so no event sits between two timed launches).

    Order: `settle_s` seconds of untimed steps (the shader clock ramps up over
    the first ~10 ms of load after the GPU idles), `warmup` untimed steps, the
    `steps` timed steps, then the same number of GEMM-only launches (the
    roofline's average launch duration), quant-only launches, and GEMM-only
    launches on one buffer set (warm: operands cached between launches)."""
    dev = torch.device("cuda:0")
    x_h = torch.from_numpy(inputs.activations(M, K, seed=0))
    w_h = torch.from_numpy(inputs.weights(N, K, seed=0))
    ops, gemm_bytes, quant_bytes = algorithmic(mode, M, N, K, gs)
    R = max(2, -(-min_set_bytes // (gemm_bytes + quant_bytes)))
    if mode in ("int8_mv", "w8a8_linear"):
        return measure_mv(cider, torch, x_h, w_h, M, N, K, gs, steps, warmup, R, ops, gemm_bytes, mode, settle_s)
    bits = 4 if mode == "w4a8" else 8
    ags = 0 if mode == "w8a8_tokpg" else gs   # activation group size
    w_dev = w_h.to(dev)
    wq0, sw0 = cider.cider_quant_weight(w_dev, bits, gs)
    del w_dev
    sets = []
    for _ in range(R):
        x = x_h.to(dev)
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        sa = torch.empty((M,) if ags == 0 else (M, K // ags), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        sets.append((x, xq, sa, wq0.clone(), sw0.clone(), y))
    # split-K workspace (scratch shared by the sets; calls run in stream order)
    ws_bytes = cider.cider_gemm_workspace_size(M, N, K, bits, gs)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # each set's two calls with their arguments marshalled once (the binding's
    # prepared calls), so that launching them costs no Python-side checking
    wsb = ws.numel() if ws is not None else 0

    def gemm_call(xq, sa, wq, sw, y):
        if mode == "w4a8":
            return cider.prepared("cider_w4a8_gemm_ex", xq, sa, wq, sw, M, N, K, y, 0, ws, wsb, stream)
        if mode == "w8a8_tokpg":
            return cider.prepared("cider_w8a8_gemm_token_group_dt", xq, sa, wq, sw, M, N, K, gs, y, 0, ws, wsb,
                                  stream)
        return cider.prepared("cider_w8a8_gemm_ex", xq, sa, wq, sw, M, N, K, gs, y, 0, ws, wsb, stream)

    calls = [(cider.prepared("cider_quant_act_dt", x, 0, M, K, ags, xq, sa, stream),
              gemm_call(xq, sa, wq, sw, y)) for (x, xq, sa, wq, sw, y) in sets]

    def timed(body):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(steps):
            body(*calls[i % R])
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    def step(quant, gemm):
        quant()
        gemm()

    settle_steps = 0
    if settle_s > 0:
        t_end = time.perf_counter() + settle_s
        while time.perf_counter() < t_end:
            for _ in range(16):
                step(*calls[settle_steps % R])
                settle_steps += 1
            torch.cuda.synchronize()
    for i in range(warmup):
        step(*calls[i % R])
    torch.cuda.synchronize()
    # the timed steps: quant + GEMM back to back, events only around the region
    step_ms = timed(step)
    # each kernel's average launch duration: the same launches, one kernel kind
    # at a time, back to back between two events on the launch stream
    g_ms = timed(lambda quant, gemm: gemm())
    q_ms = timed(lambda quant, gemm: quant())
    warm = calls[0][1]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        warm()
    end.record(stream)
    torch.cuda.synchronize()
    warm_ms = start.elapsed_time(end) / steps
    sclk = sample_sclk(torch, lambda i: calls[i % R][1](), clock_s) if clock_s > 0 else None
    del sets, calls, warm
    torch.cuda.empty_cache()
    return {"ms_per_step": step_ms, "quant_ms": q_ms, "gemm_ms": g_ms, "gemm_warm_ms": warm_ms, "ops": ops,
            "gemm_bytes": gemm_bytes, "quant_bytes": quant_bytes, "sets": R, "split_k_ws": ws_bytes,
            "sclk_mhz": sclk, "settle_steps": settle_steps}


def measure_mv(cider, torch, x_h, w_h, M, N, K, gs, steps, warmup, R, ops, nbytes, mode="int8_mv", settle_s=0.0):
    """One-launch fp16-in calls, rotating buffer sets: the decode MV (no
    activation quantization) or the one-call linear (quantization inside the
    GEMV kernel)."""
    dev = torch.device("cuda:0")
    w_dev = w_h.to(dev)
    wq0, sw0 = cider.cider_quant_weight(w_dev, 8, gs)
    del w_dev
    sets = [(x_h.to(dev), wq0.clone(), sw0.clone(), torch.empty((M, N), dtype=torch.float16, device=dev))
            for _ in range(R)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    need = cider.cider_linear_workspace_size(M, N, K, 8, gs) if mode != "int8_mv" else 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None

    def prep(x, wq, sw, y):
        if mode == "int8_mv":
            return cider.prepared("cider_int8_mv", x, wq, sw, M, N, K, gs, y, stream)
        return cider.prepared("cider_linear_dt", x, 0, wq, sw, M, N, K, 8, gs, ws, need, y, stream)

    calls = [prep(*s_) for s_ in sets]
    if settle_s > 0:
        t_end, i = time.perf_counter() + settle_s, 0
        while time.perf_counter() < t_end:
            for _ in range(64):
                calls[i % R]()
                i += 1
            torch.cuda.synchronize()
    for i in range(warmup):
        calls[i % R]()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        calls[i % R]()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del sets, calls, ws
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "quant_ms": 0.0, "gemm_ms": ms, "ops": ops, "gemm_bytes": nbytes,
            "quant_bytes": 0, "sets": R}


def measure_read_ceiling(cider, torch, nbytes=10240 * 2560, steps=200, min_set_bytes=512 * 2 ** 20):
    """The single-launch HBM read ceiling for an `nbytes` stream: cider_read_probe
    (one cold pass over a buffer, 16-byte loads, contiguous per workgroup)
    back to back over rotating buffers (>= 512 MB, so no pass finds its data
    in the 256 MB last-level cache), events around the loop."""
    dev = torch.device("cuda:0")
    R = max(2, -(-min_set_bytes // nbytes))
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(R)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    calls = [cider.prepared("cider_read_probe", b, nbytes, sink, stream) for b in bufs]
    for i in range(3 * R):
        calls[i % R]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        calls[i % R]()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del bufs, calls
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bytes": nbytes, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "kernel": "cider_read_probe",
            "note": "one launch per cold pass, back to back over rotating buffers"}


def measure_vendor(torch, M, N, K, steps=200, warmup=50):
    """Context, not a baseline: the vendor library's GEMMs at the same shape
    on the same GPU (hipBLASLt through torch): int8 x int8 -> int32
    (torch._int_mm) and fp8 e4m3 x fp8 -> fp16 with tensor scales
    (torch._scaled_mm), back to back with events on cached operands."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(0)
    a = torch.randint(-100, 100, (M, K), dtype=torch.int8, generator=g).to(dev)
    b = torch.randint(-100, 100, (N, K), dtype=torch.int8, generator=g).to(dev)
    stream = torch.cuda.current_stream()

    def timeit(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3
    out = {"note": "hipBLASLt via torch on the same GPU, warm operands; context only"}
    ops = 2.0 * M * N * K
    try:
        us = timeit(lambda: torch._int_mm(a, b.t()))
        out["int8_int32_out_us"] = round(us, 2)
        out["int8_TOPs"] = round(ops / (us * 1e-6) / 1e12, 1)
    except Exception as e:  # pragma: no cover - depends on the installed library
        out["int8_error"] = str(e)[:120]
    try:
        f8 = torch.float8_e4m3fn
        af, bf = (a.float() / 16).to(f8), (b.float() / 16).to(f8)
        one = torch.tensor(1.0, device=dev)
        us = timeit(lambda: torch._scaled_mm(af, bf.t(), scale_a=one, scale_b=one, out_dtype=torch.float16))
        out["fp8_fp16_out_us"] = round(us, 2)
        out["fp8_TOPs"] = round(ops / (us * 1e-6) / 1e12, 1)
    except Exception as e:  # pragma: no cover
        out["fp8_error"] = str(e)[:120]
    del a, b
    torch.cuda.empty_cache()
    return out


def roofline_of(ops, nbytes, ms):
    """Bound by the roof the algorithmic work hits first at peak rates."""
    t_mfma = ops / (PEAK_INT8_TOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        a = ops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(a, 3), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "frac": round(a / PEAK_INT8_TOPS, 4)}
    a = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBS, 4)}


def measure_stack(cider, torch, inputs, steps, warmup, layers=28, M=1024, dims=(2048, 2048, 1024, 6144)):
    """The chained linear stack (4 quantizations + 7 GEMMs per layer), distinct
    random weights per layer (1.4 GB of int8 codes for 28 layers: larger than
    the last-level cache, so every pass streams its weights from HBM)."""
    hidden, q_dim, kv_dim, mlp_dim = dims
    shapes = {"q": (q_dim, hidden), "k": (kv_dim, hidden), "v": (kv_dim, hidden), "o": (hidden, q_dim),
              "gate": (mlp_dim, hidden), "up": (mlp_dim, hidden), "down": (hidden, mlp_dim)}
    dev = torch.device("cuda:0")
    Ls = []
    for l in range(layers):
        L = {}
        for name, (n, k) in shapes.items():
            w = torch.from_numpy(inputs.weights(n, k, seed=inputs.stack_weight_seed(l, name))).to(dev)
            L[name] = cider.cider_quant_weight(w, 8, 0)
            del w
        Ls.append(L)
    x = torch.from_numpy(inputs.activations(M, hidden, seed=0)).to(dev)
    stream = torch.cuda.current_stream()

    def timed(layers_):
        y, ws = cider.cider_stack_forward(x, layers_, dims)
        for _ in range(warmup):
            cider.cider_stack_forward(x, layers_, dims, workspace=ws, y=y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            cider.cider_stack_forward(x, layers_, dims, workspace=ws, y=y, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_sep = timed(Ls)
    # the same weights with q/k/v and gate/up adjacent: one GEMM per group
    Ls = [cider.fuse_stack_layer(L) for L in Ls]
    torch.cuda.empty_cache()
    ms = timed(Ls)
    ops = 2.0 * M * layers * sum(n * k for n, k in shapes.values())
    del Ls
    torch.cuda.empty_cache()
    return {"workload": f"{layers}-layer linear stack, seq {M}, hidden {hidden}, q {q_dim}, kv {kv_dim}, "
                        f"mlp {mlp_dim}: {4 * layers} quantizations + {4 * layers} GEMMs per pass "
                        f"(q/k/v and gate/up fused)",
            "ms_per_pass": round(ms, 4), "TOP/s": round(ops / (ms * 1e-3) / 1e12, 2), "ops_per_pass": ops,
            "ms_per_pass_unfused": round(ms_sep, 4), "steps": steps}


SWEEP = ([("w8a8_pc", M, 10240, 2560, 0) for M in (1, 128, 1024, 4096, 8192)] +
         [("w8a8_pc", M, 2560, 10240, 0) for M in (1, 128, 1024, 4096, 8192)] +
         [("w8a8_pg", M, 2560, 10240, gs) for gs in (128, 64) for M in (128, 1024, 4096)] +
         [("w8a8_tokpg", M, 2560, 10240, gs) for gs in (128, 64) for M in (16, 128, 1024, 4096)] +
         [("w4a8", M, 10240, 2560, 0) for M in (1, 1024, 8192)] +
         [("int8_mv", 1, 10240, 2560, 0), ("int8_mv", 1, 2560, 10240, 0), ("int8_mv", 1, 10240, 2560, 128),
          ("int8_mv", 1, 2560, 10240, 128), ("int8_mv", 1, 2560, 10240, 64)] +
         [("w8a8_linear", 1, 10240, 2560, 0), ("w8a8_linear", 1, 2560, 10240, 0), ("w8a8_linear", 4, 10240, 2560, 0)])


def sweep_indices(spec):
    """Sweep row indices from "3", "0-4,9" or "" (all rows)."""
    if not spec:
        return list(range(len(SWEEP)))
    out = []
    for part in spec.split(","):
        a, _, b = part.partition("-")
        out.extend(range(int(a), int(b or a) + 1))
    if any(i < 0 or i >= len(SWEEP) for i in out):
        raise SystemExit(f"--sweep-rows: indices must lie in 0..{len(SWEEP) - 1}")
    return out


VALU_LANE_OPS_PER_S = 256 * 64 * 2.4e9   # non-packed fp32 VALU: 64 lane-ops per clock per CU


def pg_coroof(mode, M, N, K, gs, ops, us):
    """Per-group's second roof: the fp32 fold after every group is VALU work
    the matrix cores do not do: cvt + mul + fma per output element and group
    (both scales per group), cvt + fma with per-token activation scales. The
    co-roof is max(MFMA time, fold VALU time) at peak rates."""
    G = K // gs
    fold = (3 if mode == "w8a8_pg" else 2) * M * N * G
    t_valu = fold / VALU_LANE_OPS_PER_S * 1e6
    t_mfma = ops / (PEAK_INT8_TOPS * 1e12) * 1e6
    co = max(t_valu, t_mfma)
    return {"fold_lane_ops": fold, "t_valu_us": round(t_valu, 2), "t_mfma_us": round(t_mfma, 2),
            "co_roof_us": round(co, 2), "frac_of_co_roof": round(co / us, 4)}


def run_sweep(cider, torch, inputs, indices, steps, settle_s=0.0):
    """Times the selected sweep configurations, each with its own roofline
    (each row first runs settle_s seconds of untimed launches, so that a
    profiled single-row run sees the same settled clock as the headline)."""
    rows = []
    for i in indices:
        mode, m, n, k, gs = SWEEP[i]
        rr = measure(cider, torch, inputs, mode, m, n, k, gs, max(10, steps // 2), max(3, steps // 4),
                     settle_s=settle_s)
        rows.append({"row": i, "mode": mode, "M": m, "N": n, "K": k, "group_size": gs,
                     "gemm_us": round(rr["gemm_ms"] * 1e3, 2), "quant_us": round(rr["quant_ms"] * 1e3, 2),
                     "gemm_roofline": roofline_of(rr["ops"], rr["gemm_bytes"], rr["gemm_ms"]),
                     "quant_GBs": round(rr["quant_bytes"] / (rr["quant_ms"] * 1e-3) / 1e9, 1) if rr["quant_ms"] else None,
                     "linear_TOPs": round(rr["ops"] / (rr["ms_per_step"] * 1e-3) / 1e12, 2),
                     "split_k": bool(rr.get("split_k_ws"))})
        if mode in ("w8a8_pg", "w8a8_tokpg"):
            rows[-1]["valu_co_roof"] = pg_coroof(mode, m, n, k, gs, rr["ops"], rr["gemm_ms"] * 1e3)
        print(json.dumps({"sweep_row": rows[-1]}), file=sys.stderr, flush=True)
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: ~11 ms of untimed steps, then ~23 ms timed. The shader clock
    # ramps up over the first ~10 ms of sustained load after an idle GPU, so
    # every run first settles for --settle-ms of untimed steps (5 warm-up
    # steps alone timed that ramp: step 130 us instead of 113 us)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps run for this long before the warm-up steps (clock ramp)")
    ap.add_argument("--clock-s", type=float, default=1.0,
                    help="seconds of back-to-back GEMMs during which the shader clock is read from "
                         "sysfs after the timed loops (0: no sampling)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock sampling (also skipped automatically under rocprofv3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="also time every per-channel / per-group / W4A8 configuration")
    ap.add_argument("--stack", action="store_true",
                    help="also time the 28-layer Qwen3-VL-2B-shaped linear stack at seq 1024")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--sweep-rows", default="",
                    help="with --sweep / --sweep-only: indices of the sweep rows to run, e.g. 3 or 0-4,9")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="also measure the single-launch HBM read ceiling of a 26.2 MB stream "
                         "(the M=1 weight stream), also done with --sweep")
    ap.add_argument("--vendor", action="store_true",
                    help="also time the vendor library's int8 and fp8 GEMMs at the headline shape (context)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="run only the sweep rows (no headline step, no CPU baseline): one JSON line "
                         "with the rows, for per-configuration profiler runs")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(collectives and sharding are out of scope); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from w8a8_online_quantized_amd import cider, inputs

    if not torch.cuda.is_available() or not cider.cider_is_available():
        print("bench.py needs a gfx950 GPU and the built libcider.so", file=sys.stderr)
        sys.exit(3)

    if args.sweep_only:
        rows = run_sweep(cider, torch, inputs, sweep_indices(args.sweep_rows), args.steps,
                         settle_s=args.settle_ms * 1e-3)
        res = {"sweep": rows, "kernel_source_sha": kernel_source_sha()}
        if args.read_ceiling:
            res["read_ceiling"] = measure_read_ceiling(cider, torch)
        print(json.dumps(res), flush=True)
        return

    M, N, K = 4096, 10240, 2560
    clock_s = 0.0 if (args.no_clock or profiler_attached()) else args.clock_s
    r = measure(cider, torch, inputs, "w8a8_pc", M, N, K, 0, args.steps, args.warmup, clock_s=clock_s,
                settle_s=args.settle_ms * 1e-3)
    ops = r["ops"]
    value = ops / (r["ms_per_step"] * 1e-3) / 1e12
    gemm_tops = ops / (r["gemm_ms"] * 1e-3) / 1e12

    if args.calib_copy_mb:
        n = args.calib_copy_mb * 2 ** 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    sha = kernel_source_sha()
    out = {
        "metric": "Fused W8A8 GEMM TOPS at M=4096,N=10240,K=2560; % of INT8 MFMA peak",
        "value": round(value, 3),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_M5PRO_TOPS, 3),
        "dtype": "i8",
        "data": "synthetic",
        "settle": {"ms": args.settle_ms, "steps": r["settle_steps"],
                   "note": "untimed steps before the warm-up steps while the shader clock ramps up"},
        "config": {"workload": f"w8a8 per-channel online-quantized linear, M={M} N={N} K={K}, "
                               f"quant_act + fused GEMM per step",
                   "M": M, "N": N, "K": K, "group_size": 0, "x_dtype": "fp16", "y_dtype": "fp16",
                   "cold_cache_sets": r["sets"], "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "cider_w8a8_gemm",
                     "achieved": round(gemm_tops, 3), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": measured_traffic(sha),
                     "algorithmic_bytes": r["gemm_bytes"], "algorithmic_ops": ops,
                     "avg_launch_ms": round(r["gemm_ms"], 5),
                     "avg_launch_source": f"HIP events around {args.steps} back-to-back cider_w8a8_gemm "
                                          f"launches (rotating {r['sets']} buffer sets) on the launch stream, "
                                          f"right after the timed steps",
                     "warm_launch_ms": round(r["gemm_warm_ms"], 5),
                     "warm_note": "the same GEMM relaunched on one buffer set (operands stay cached): warm",
                     # shader clock read from sysfs (no process spawned) while the GEMM ran back
                     # to back after the timed loops: median, min, max, samples; and the
                     # fraction of the dense peak at the median clock
                     "sclk_mhz": ({"median": round(r["sclk_mhz"][0]), "min": round(r["sclk_mhz"][1]),
                                   "max": round(r["sclk_mhz"][2]), "samples": r["sclk_mhz"][3]}
                                  if r["sclk_mhz"] else None),
                     "mclk_mhz": (round(r["sclk_mhz"][4]) if r["sclk_mhz"] and r["sclk_mhz"][4] else None),
                     "frac_at_sclk": (round(gemm_tops / (PEAK_INT8_TOPS * r["sclk_mhz"][0] / 2400.0), 4)
                                      if r["sclk_mhz"] else None)},
        "kernels": {"cider_quant_act": {"avg_ms": round(r["quant_ms"], 5),
                                        "GB/s": round(r["quant_bytes"] / (r["quant_ms"] * 1e-3) / 1e9, 1),
                                        "hbm_frac": round(r["quant_bytes"] / (r["quant_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                    "cider_w8a8_gemm": {"avg_ms": round(r["gemm_ms"], 5), "TOP/s": round(gemm_tops, 2)}},
        "baseline_context": f"Apple M5 Pro, README single-op table: 4.41 ms = {PAGES_M5PRO_TOPS:.1f} TOP/s",
        "kernel_source_sha": sha,
    }
    if args.sweep:
        out["sweep"] = run_sweep(cider, torch, inputs, sweep_indices(args.sweep_rows), args.steps,
                                 settle_s=args.settle_ms * 1e-3)
    if args.sweep or args.read_ceiling:
        out["read_ceiling"] = measure_read_ceiling(cider, torch)
    if args.vendor:
        out["vendor_reference"] = measure_vendor(torch, M, N, K)
    if args.stack:
        out["stack"] = measure_stack(cider, torch, inputs, max(3, args.steps // 10), 3)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(M, N, K)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
