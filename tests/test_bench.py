"""The benchmark harness's host-side logic, on the CPU: the one-GPU guard, the traffic lookup that
must go null when a kernel's sources change, and the time-based warm-up."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_recorded_sources(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    name, ent = next(iter(rec["kernels"].items()))
    if ent["sources_sha256"] == bench.kernel_sources_digest(ent["sources"]):
        assert bench.measured_traffic(name) == ent["hbm_bytes_per_launch"]
    # any change to the kernel's sources voids the figure
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda names: "0" * 64)
    assert bench.measured_traffic(name) is None
    assert bench.measured_traffic("no_such_kernel") is None


def test_warm_up_runs_for_its_time_and_at_least_its_calls():
    class FakeTorch:
        class cuda:
            syncs = 0

            @staticmethod
            def synchronize():
                FakeTorch.cuda.syncs += 1

    calls = []
    n = bench.warm_up(FakeTorch, lambda: calls.append(1), seconds=0.0, min_calls=5)
    assert n == len(calls) == 5 and FakeTorch.cuda.syncs >= 1
    calls.clear()
    n = bench.warm_up(FakeTorch, lambda: calls.append(1), seconds=0.05, min_calls=1)
    assert n == len(calls) >= 1
