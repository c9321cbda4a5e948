"""bench.py's host-side logic, on the CPU: the refusal of more than one GPU,
the roofline choice and its algorithmic bytes and ops, sweep-row parsing, the
per-group VALU co-roof, the sysfs clock parser, profiler detection, and the
gate that reports committed counter traffic only for the kernel sources it
was taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_and_ops():
    M, N, K = 4096, 10240, 2560
    ops, gb, qb = bench.algorithmic("w8a8_pc", M, N, K, 0)
    assert ops == 2.0 * M * N * K
    assert gb == M * K + N * K + 4 * M + 4 * N + 2 * M * N == 120643584
    assert qb == 2 * M * K + M * K + 4 * M
    # per-group: one scale per row (column) and group on both sides
    _, gb, qb = bench.algorithmic("w8a8_pg", 128, 2560, 10240, 128)
    assert gb == 128 * 10240 + 2560 * 10240 + 4 * 128 * 80 + 4 * 2560 * 80 + 2 * 128 * 2560
    assert qb == 3 * 128 * 10240 + 4 * 128 * 80
    # per-token activations x per-group weights: one activation scale per row
    _, gb, _ = bench.algorithmic("w8a8_tokpg", 128, 2560, 10240, 128)
    assert gb == 128 * 10240 + 2560 * 10240 + 4 * 128 + 4 * 2560 * 80 + 2 * 128 * 2560
    # int4 weights: half a byte per code
    _, gb, _ = bench.algorithmic("w4a8", 1, 10240, 2560, 0)
    assert gb == 2560 + 10240 * 2560 // 2 + 4 + 4 * 10240 + 2 * 10240
    # one-launch fp16-in paths: fp16 x, no quantization pass
    _, gb, qb = bench.algorithmic("int8_mv", 1, 10240, 2560, 0)
    assert gb == 2 * 2560 + 10240 * 2560 + 4 * 10240 + 2 * 10240 and qb == 0


def test_roofline_picks_the_roof_the_work_hits_first():
    # the headline is above the ridge (629 ops per byte): MFMA-bound
    ops, gb, _ = bench.algorithmic("w8a8_pc", 4096, 10240, 2560, 0)
    r = bench.roofline_of(ops, gb, 0.0859)
    assert r["bound"] == "mfma" and r["unit"] == "TOP/s"
    assert r["frac"] == pytest.approx(ops / 0.0859e-3 / 1e12 / 5000.0, abs=1e-4)
    # M = 1 is far below it: HBM-bound
    ops, gb, _ = bench.algorithmic("w8a8_pc", 1, 10240, 2560, 0)
    r = bench.roofline_of(ops, gb, 0.0072)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(gb / 0.0072e-3 / 1e9 / 8000.0, abs=1e-4)


def test_sweep_row_parsing():
    n = len(bench.SWEEP)
    assert bench.sweep_indices("") == list(range(n))
    assert bench.sweep_indices("3") == [3]
    assert bench.sweep_indices("0-4,9") == [0, 1, 2, 3, 4, 9]
    with pytest.raises(SystemExit):
        bench.sweep_indices(str(n))


def test_per_group_co_roof():
    M, N, K, gs = 4096, 2560, 10240, 128
    ops = 2.0 * M * N * K
    r = bench.pg_coroof("w8a8_pg", M, N, K, gs, ops, 150.0)
    assert r["fold_lane_ops"] == 3 * M * N * (K // gs)
    t_valu = 3 * M * N * (K // gs) / (256 * 64 * 2.4e9) * 1e6
    t_mfma = ops / 5e15 * 1e6
    assert r["co_roof_us"] == pytest.approx(max(t_valu, t_mfma), abs=0.01)
    assert r["frac_of_co_roof"] == pytest.approx(max(t_valu, t_mfma) / 150.0, abs=1e-4)
    # per-token activation scales: cvt + fma only
    assert bench.pg_coroof("w8a8_tokpg", M, N, K, gs, ops, 150.0)["fold_lane_ops"] == 2 * M * N * (K // gs)


def test_dpm_table_parser(tmp_path):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text("0: 500Mhz\n1: 1600Mhz\n2: 2083Mhz *\n")
    assert bench._read_dpm_mhz(str(p)) == 2083.0
    p.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench._read_dpm_mhz(str(p)) is None
    assert bench._read_dpm_mhz(str(tmp_path / "missing")) is None


def test_profiler_detection(monkeypatch):
    for k in [k for k in os.environ if k.startswith("ROCPROF")]:
        monkeypatch.delenv(k)
    monkeypatch.setenv("LD_PRELOAD", "")
    assert not bench.profiler_attached()
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/librocprofiler-sdk-tool.so")
    assert bench.profiler_attached()
    monkeypatch.setenv("LD_PRELOAD", "")
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp/x")
    assert bench.profiler_attached()


def test_traffic_reported_only_for_the_kernel_sources_it_was_taken_on(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel_source_sha": "abc", "bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("abc") == 123
    assert bench.measured_traffic("def") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("abc") is None
