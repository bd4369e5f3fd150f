"""Host-side checks of bench.py (no GPU): the one-GPU guard, the traffic
record lookup, the repeatability counter and the host record."""

import os
import subprocess
import sys

import torch

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_only_for_its_own_run():
    # the committed counter record covers one workload, schedule and protocol
    assert bench.measured_traffic("C3", "shift", "auto") is None
    assert bench.measured_traffic("C2", "naive", "auto") is None
    assert bench.measured_traffic("C2", "shift", "device") is None
    t = bench.measured_traffic("C2", "shift", "auto")
    assert t is None or t > 2.0e8  # at least the compulsory bytes of C2 when the sources match


def test_repeat_check_counts_identical_runs():
    a = torch.arange(12, dtype=torch.bfloat16)
    assert bench.repeat_check(lambda: (a, a, a), 20, torch) == 20
    calls = {"n": 0}

    def flaky():
        calls["n"] += 1
        b = a.clone()
        if calls["n"] % 2 == 0:
            b[3] = -b[3]
        return (a, b, a)

    assert bench.repeat_check(flaky, 20, torch) == 10


def test_host_info_fields():
    h = bench.host_info(torch)
    assert set(h) == {"cpu_model", "cpu_threads", "hip", "torch", "gpu"}
    assert h["cpu_threads"] >= 1
