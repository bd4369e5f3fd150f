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
    # each committed counter record covers one workload, schedule and protocol
    assert bench.measured_traffic("C1", "shift", "auto") is None
    assert bench.measured_traffic("C3", "shift", "device") is None
    for w, compulsory in (("C3", 1.0e9), ("C3F", 1.0e9)):
        for s in ("shift", "descending"):
            t = bench.measured_traffic(w, s, "auto")
            assert t is None or t > compulsory  # at least the compulsory bytes when the sources match


def _counter_csv(path, counter, rows):
    import csv
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, value) in enumerate(rows):
            wr.writerow([i + 1, name, counter, value])


def test_make_traffic_record_arithmetic(tmp_path, monkeypatch):
    # two main-kernel dispatches and three 1 GiB copies per run: FETCH_SIZE reads 524288 KiB
    # on a copy (scale 2), WRITE_SIZE 1048576 KiB (scale 1)
    main = "void attn::bwd_main_kernel<128, 128, 64, true, 2>(attn::MainParams)"
    copy = "void at::native::copy_kernel(...)"
    _counter_csv(tmp_path / "f", "FETCH_SIZE", [(main, 1000.0), (main, 3000.0), (copy, 524288.0), (copy, 524288.0),
                                                (copy, 524288.0)])
    _counter_csv(tmp_path / "w", "WRITE_SIZE", [(main, 500.0), (main, 500.0), ("other", 7.0), (copy, 1048576.0),
                                                (copy, 1048576.0), (copy, 1048576.0)])
    out = tmp_path / "rec.json"
    monkeypatch.setattr(bench, "traffic_path", lambda w, s: str(out))
    args = bench.argparse.Namespace(make_traffic_record=(str(tmp_path / "f"), str(tmp_path / "w")),
                                    workload="C3", schedules="shift", dq_protocol="auto")
    bench.make_traffic_record(args)
    import json
    rec = json.load(open(out))
    assert rec["fetch_bytes"] == 2000 * 1024 * 2
    assert rec["write_bytes"] == 500 * 1024
    assert rec["traffic_bytes"] == 2000 * 1024 * 2 + 500 * 1024
    assert rec["schedule"] == "shift" and rec["workload"].startswith("C3:")
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()


def test_source_hash_ignores_comments_and_layout_only():
    src = 'int a = 1; // note\n/* block\n comment */  asm volatile("s_waitcnt vmcnt(0) // kept" ::: "memory");\n'
    assert bench.code_only(src) == 'int a = 1; asm volatile("s_waitcnt vmcnt(0) // kept" ::: "memory");'
    assert bench.code_only(src) == bench.code_only(src.replace("// note", "// other words").replace("  ", "\n\t"))
    assert bench.code_only(src) != bench.code_only(src.replace("a = 1", "a = 2"))
    texts = {f: open(os.path.join(ROOT, "deterministic_attention_backward_amd", "csrc", f)).read()
             for f in bench.KERNEL_SOURCES}
    h = bench.kernel_source_hash(lambda f: texts[f])
    assert h == bench.kernel_source_hash()
    first = bench.KERNEL_SOURCES[0]
    assert bench.kernel_source_hash(lambda f: texts[f] + ("// x\n" if f == first else "")) == h
    assert bench.kernel_source_hash(lambda f: texts[f] + ("int z;\n" if f == first else "")) != h


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
