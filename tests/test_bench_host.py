"""Host logic of bench.py (no GPU): the one-GPU contract, the throughput
arithmetic, and the rule that counter traffic is reported only for the
kernel sources it was measured on."""
import json
import os

import pytest

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    err = capsys.readouterr().err
    assert "ONE GPU" in err and "--gpus 1" in err


def test_no_gpu_is_an_error_not_a_fallback(capsys):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the benchmark would run")
    assert bench.main([]) == 1
    assert "needs a GPU" in capsys.readouterr().err


def test_row_entry_arithmetic():
    e = bench.row_entry(8_000_000_000, 1000.0)   # 8 GB in 1000 ms
    assert e["us"] == 1_000_000.0
    assert e["gbs"] == 8.0 and e["frac"] == round(8.0 / 8000.0, 4)
    e = bench.row_entry(268_435_456, 0.0465, cpu_bytes=268_435_456, cpu_s=0.004, note="x")
    assert abs(e["gbs"] - 268_435_456 / 46.5e-6 / 1e9) < 0.1
    assert abs(e["oracle_gbs"] - 268_435_456 / 0.004 / 1e9) < 1e-3 and e["oracle_sample"] == "x"


def test_stored_traffic_is_consistent():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    alg = rec["algorithmic_bytes_per_launch"]
    assert alg == 2 * 4 * 32 * 2 ** 20          # W=4 x 32 MiB read + written
    assert abs(rec["hbm_bytes_per_launch"] / alg - 1) < 0.01
    assert abs(rec["copy_only_kernel_hbm_bytes_per_launch"] / alg - 1) < 0.01
    assert abs(rec["plain_copy_kernel_hbm_bytes_per_launch"] / alg - 1) < 0.01


def test_traffic_is_dropped_when_the_kernel_changes(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    src = tmp_path / "a2av.hip"
    src.write_text("// a different kernel\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    assert bench.kernel_source_hash() != rec["kernel_source_hash"]
    assert bench.traffic_entry(rec["algorithmic_bytes_per_launch"]) is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["kernel_source_hash"])
    assert bench.traffic_entry(rec["algorithmic_bytes_per_launch"]) == rec["hbm_bytes_per_launch"]
