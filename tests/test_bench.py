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


def test_distribution_summary():
    d = bench.dist([3.0, 1.0, 2.0, 4.0, 5.0])
    assert d["n"] == 5 and d["median_ms"] == 3.0 and d["min_ms"] == 1.0 and d["max_ms"] == 5.0
    assert d["p10_ms"] == 1.4 and abs(d["p90_ms"] - 4.6) < 1e-12 and d["mean_ms"] == 3.0
    assert bench.dist([]) == {"n": 0}


def test_host_record_names_the_cpus():
    h = bench.host_record()
    assert h["affinity_cpus"] >= 1 and h["cpu_model"]
    assert h["numa_nodes"] is None or h["numa_nodes"] >= 1


def test_rates_against_peak_and_ceiling():
    ceil = {"mfma_bf16_tflops": 2000.0, "mfma_fp8_tflops": 4000.0, "hbm_read_gbs": 7000.0}
    r = bench.rate_of("mfma", 2.5e12, 1.0, ceil)  # 2.5 TFLOP in 1 ms
    assert abs(r["tflops"] - 2500.0) < 1e-9 and abs(r["frac_of_ceiling"] - 1.25) < 1e-12
    assert "frac_of_data_ceiling" not in r  # no data-dependent ceiling given
    r = bench.rate_of("mfma", 2.5e12, 1.0, dict(ceil, mfma_bf16_random_tflops=1250.0))
    assert abs(r["frac_of_data_ceiling"] - 2.0) < 1e-12
    r = bench.rate_of("hbm", 7e9, 1.0, ceil)  # 7 GB in 1 ms
    assert abs(r["gbs"] - 7000.0) < 1e-9 and abs(r["frac_of_peak"] - 0.875) < 1e-12


def test_committed_ceilings_without_measuring():
    c = bench.ceilings(False)
    assert c["mfma_bf16_tflops"] > 2000 and c["hbm_read_gbs"] > 6000 and "committed" in c["source"]


def test_leg_time_source_and_rates():
    """A leg's time per call: the back-to-back loop when there is one, else the per-call events (legs
    with work between calls); the library timer's per-kernel durations are kept apart and never set
    the rate."""
    ceil = dict(bench.COMMITTED_CEILINGS)
    base = {"per_call": [0.5] * 20 + [0.6] * 5, "per_kernel": {"k": [0.9] * 25}}
    loop = bench.leg_record({**base, "wall_s": 0.02, "loop_ms": 10.0}, 25, "mfma", 1e12, ceil, "k")
    assert loop["time_source"] == "back-to-back loop" and loop["avg_ms"] == 10.0 / 25
    assert abs(loop["tflops"] - 1e12 / 0.4e-3 / 1e12) < 1e-9
    assert loop["kernels_sum_ms"] == 0.9 and loop["loop_ms_per_call"] == 0.4
    events = bench.leg_record({**base, "wall_s": None, "loop_ms": None}, 25, "hbm", 1e9, ceil)
    assert events["time_source"] == "per-call events"
    assert abs(events["avg_ms"] - (20 * 0.5 + 5 * 0.6) / 25) < 1e-12 and "loop_ms_per_call" not in events
    assert abs(events["gbs"] - 1e9 / (events["avg_ms"] * 1e-3) / 1e9) < 1e-9


def test_roofline_time_names_the_binding_resource():
    from roofline_attention_amd import ledger as L
    # [4,16,1024,64] causal bf16: 8.6 GFLOP (3.4 us at the bf16 peak) but 33.8 MB of compulsory
    # traffic (4.2 us at 8 TB/s), so the HBM bound sets its roofline
    fl = L.fwd_flops(4, 16, 1024, 64, True)
    by = L.fwd_bytes(4, 16, 16, 1024, 64, 2)
    r = bench.roofline_time(fl, L.PEAK_BF16_TFLOPS, by, 0.0184)
    assert r["bound"] == "hbm"
    assert abs(r["hbm_ms"] - by / 8e12 * 1e3) < 1e-12 and r["hbm_ms"] > r["mfma_ms"]
    assert abs(r["frac"] - r["hbm_ms"] / 0.0184) < 1e-12
    # [2,32,4096,128] causal: compute-bound
    r = bench.roofline_time(L.fwd_flops(2, 32, 4096, 128, True), L.PEAK_BF16_TFLOPS,
                            L.fwd_bytes(2, 32, 32, 4096, 128, 2), 0.26)
    assert r["bound"] == "mfma" and 0.4 < r["frac"] < 0.45
