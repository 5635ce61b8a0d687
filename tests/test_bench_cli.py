"""Host logic of bench.py that runs without a GPU: the one-GPU contract and
the lookup of committed counter records."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_a_launcher_world_size_above_one_is_refused(monkeypatch, capsys):
    monkeypatch.setenv("WORLD_SIZE", "4")
    assert bench.main([]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU path")
def test_no_gpu_no_number(capsys):
    """Without a GPU the bench prints no JSON line and fails: there is no CPU
    stand-in for the measured path."""
    assert bench.main(["--no-cpu-baseline"]) == 2
    out = capsys.readouterr()
    assert "needs a GPU" in out.err and not out.out.strip()


def test_counter_records_only_for_known_kernels_and_workloads():
    assert bench.counter_record("f16_4096x4096x8192", "no_such_kernel") is None
    assert bench.counter_record("no_such_workload", "pipelined") is None


def test_counter_record_follows_the_kernel_code(tmp_path, monkeypatch):
    """A record is reported only while its code hash is the kernel's current
    one: a record taken on other code gives None (traffic null in the line)."""
    from matrix_core_scheduling_amd import profiling

    key = profiling.traffic_key("f16_4096x4096x8192", "pipelined")
    rec = {"fetch_bytes_per_launch": 1, "write_bytes_per_launch": 1, "hbm_bytes_per_launch": 2,
           "mfma_busy": 0.5, "clock_GHz": 1.0, "fetch_scale": 2.0, "write_scale": 1.0,
           "copy_calibration_mib": 256}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({key: dict(rec, kernel_code_sha256=profiling.kernel_code_hash("pipelined"))}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.counter_record("f16_4096x4096x8192", "pipelined")["hbm_bytes_per_launch"] == 2
    f.write_text(json.dumps({key: dict(rec, kernel_code_sha256="0" * 64)}))
    assert bench.counter_record("f16_4096x4096x8192", "pipelined") is None
