"""bench.py on the CPU: the one-GPU contract and the source-hash rule of the committed traffic counters."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (module import only: no GPU work happens at import time)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_kernel_sources_exist():
    for kernel, paths in bench.KERNEL_SOURCES.items():
        for p in paths:
            assert os.path.exists(os.path.join(ROOT, p)), f"{kernel}: {p}"


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        data = json.load(f)
    cal = data["calibration"]
    assert cal["fetch_factor"] > 0 and cal["write_factor"] > 0
    keys = [k for k in data if k != "calibration"]
    assert keys
    for key in keys:
        kernel, workload = key.split(":")
        ent = data[key]
        got = bench.traffic_from_profile(kernel, workload)
        if ent["source_sha"] == bench.sha_of(bench.KERNEL_SOURCES[kernel]):
            want = 1024.0 * (ent["fetch_kib"] * cal["fetch_factor"] + ent["write_kib"] * cal["write_factor"])
            assert got == want
        else:
            assert got is None
    # any change of a kernel's sources makes its figure stale
    monkeypatch.setattr(bench, "sha_of", lambda paths: "0" * 16)
    for key in keys:
        kernel, workload = key.split(":")
        assert bench.traffic_from_profile(kernel, workload) is None
    assert bench.traffic_from_profile("gemm", "no_such_workload") is None
