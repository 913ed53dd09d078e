"""Host logic of bench.py (no GPU): the one-GPU guard, the code-only source
hash behind the stored traffic counters, and the counter calibration."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_code_only_ignores_comments_and_spacing():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* no overflow\n check */\n}\n"
    b = "int f(int x) {\n\n    return 2 * x;\n}   // edited comment\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    # text inside an inline-asm string is code
    assert "global_load_lds_dwordx4" in bench._code_only('asm volatile("global_load_lds_dwordx4 %1, %2");')


def _counter_csv(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_traffic_calibration(tmp_path):
    gib_kib = 1 << 20
    # the copy reads half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    _counter_csv(tmp_path / "cf", [(1, "copyBuffer", "FETCH_SIZE", gib_kib / 2), (2, "small", "FETCH_SIZE", 10)])
    _counter_csv(tmp_path / "cw", [(1, "copyBuffer", "WRITE_SIZE", gib_kib)])
    # two dispatches per kernel; one counter row split over two instances for the second
    _counter_csv(tmp_path / "f", [(5, "k_fwd_big<Cfg>(P)", "FETCH_SIZE", 1000), (6, "k_fwd_big<Cfg>(P)", "FETCH_SIZE", 600),
                                  (6, "k_fwd_big<Cfg>(P)", "FETCH_SIZE", 400), (7, "k_dx_big<Cfg>(P)", "FETCH_SIZE", 2000),
                                  (8, "k_dx_big<Cfg>(P)", "FETCH_SIZE", 2000), (9, "k_other", "FETCH_SIZE", 9e9)])
    _counter_csv(tmp_path / "w", [(5, "k_fwd_big<Cfg>(P)", "WRITE_SIZE", 300), (6, "k_fwd_big<Cfg>(P)", "WRITE_SIZE", 500),
                                  (7, "k_dx_big<Cfg>(P)", "WRITE_SIZE", 700), (8, "k_dx_big<Cfg>(P)", "WRITE_SIZE", 700)])
    out = tmp_path / "traffic.json"
    bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                        path=str(out))
    data = json.loads(out.read_text())
    assert data["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert data["calibration"]["write_factor"] == pytest.approx(1.0)
    fwd, dx = data["fwd_gemm"], data["bwd_dx_gemm"]
    assert fwd["fetch_kib_per_dispatch"] == pytest.approx(1000)   # (1000 + (600 + 400)) / 2
    assert fwd["write_kib_per_dispatch"] == pytest.approx(400)
    assert fwd["bytes_per_launch"] == pytest.approx(1024 * (1000 * 2 + 400))
    assert dx["bytes_per_launch"] == pytest.approx(1024 * (2000 * 2 + 700))
    assert fwd["source_hash"] == bench.kernel_source_hash("fwd_gemm")
