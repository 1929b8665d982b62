"""Host logic of bench.py (no GPU): the one-GPU contract, the algorithmic byte
count, the source-hash guard on stored traffic measurements and the
PMC-calibration arithmetic."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_weight_bytes_is_codes_scales_and_g():
    # the square projection: N*K/2 code bytes, N*K/16 E4M3 scale bytes, one fp32 g
    assert bench.weight_bytes(5120, 5120) == 13_107_200 + 1_638_400 + 4
    assert bench.weight_bytes(17408, 5120) == 17408 * 2560 + 17408 * 320 + 4


def test_stored_traffic_only_for_the_sources_it_was_taken_on(monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        stored = json.load(f)
    if stored["kernel_source_hash"] == bench.kernel_source_hash():
        assert bench.stored_traffic() == stored["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.stored_traffic() is None


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, ctr, v in rows:
            f.write(f'"{name}",{ctr},{v}\n')


def test_ingest_pmc_scales_each_counter_by_the_copy(tmp_path, monkeypatch):
    d = tmp_path / "pmc"
    # the copy of 256 MiB reads as twice its bytes on FETCH_SIZE and as its
    # bytes on WRITE_SIZE; the GEMV's dispatches read 7000 / 7200 / 7100 KiB
    _counter_csv(str(d / "pmc_copy_FETCH_SIZE"), [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 2 * 262144)])
    _counter_csv(str(d / "pmc_copy_WRITE_SIZE"), [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 262144)])
    _counter_csv(str(d / "pmc_bench_FETCH_SIZE"),
                 [("void w4a16::k_gemm_rows<1, 5, 0>(w4a16::MatArgs)", "FETCH_SIZE", v) for v in (7000, 7200, 7100)]
                 + [("void at::native::fill", "FETCH_SIZE", 999999)])
    _counter_csv(str(d / "pmc_bench_WRITE_SIZE"),
                 [("void w4a16::k_gemm_rows<1, 5, 0>(w4a16::MatArgs)", "WRITE_SIZE", 16)])
    out_file = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out_file))
    bench.ingest_pmc(str(d))
    t = json.loads(out_file.read_text())
    assert t["FETCH_SIZE"]["factor"] == 0.5 and t["WRITE_SIZE"]["factor"] == 1.0
    # median 7100 KiB at half the counter's reading, plus 16 KiB written
    assert t["bytes_per_launch"] == 7100 * 512 + 16 * 1024
    assert t["algorithmic_bytes_per_launch"] == bench.weight_bytes(5120, 5120)
    assert t["kernel_source_hash"] == bench.kernel_source_hash()
