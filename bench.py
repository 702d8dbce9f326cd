"""Benchmark of the attention hot path on one MI355X.

A step is one forward + backward pass (attn_fwd then attn_bwd, all forward and backward kernels)
of causal bf16 attention over the [B=2, H=16, N=4096, d=128] synthetic batch, inputs resident in
HBM before timing starts. The decode kernels and the prefill forwards are timed as extra legs in
the same run and reported beside the step. Every timed region runs three passes of its calls: back
to back with events only at the loop's two ends (the throughput figure), with an event pair on the
launch stream around each call (the per-call distribution: median, p10, p90, minimum), and with the
library's timer on, whose events around every kernel give each kernel's launch durations ("M4.2 -
GPU Execution Model for Transformer Kernels", section 0x0B, Level 4: report a median and a tail,
not one timing). The launch-bound 1k prefill is also replayed from a HIP graph of its calls, for
comparison (a graph takes the host's launch cost out). Rates are priced against the published MI355X peaks
and against ceilings measured on the same GPU in the same run ("Why Fast GPUs Still Wait for
Memory", section "pi is the top of a stack": measure your own ceilings before trusting them).

Output: one JSON line on stdout (rank 0), with the roofline of the dominant kernel and the fp64
CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--legs/--no-legs]
                       [--no-ceilings]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd/bwd TFLOP/s and decode HBM GB/s, % of MI355X roofline"
WARMUP_S = 0.2  # untimed seconds of load before every timed region (the clock ramps up first)
LEG_CALLS = 30  # timed calls per leg and pass (>= 20 samples each)
GRAPH_REPLAYS = 20  # timed replays of a graph of LEG_CALLS calls (launch-bound legs)

# Ceilings measured by the ceiling microbenchmarks (csrc/ceilings.hip) on one MI355X, used only when
# the executable is not available in this run: dense bf16 and E4M3 MFMA on the full chip after a
# warm-up, on operands that barely switch (the same small values in every lane) and on operands
# like the kernels' (random full-mantissa values, a new pair each instruction; under the chip's
# power management the clock, and with it the rate, depends on the data), and the HBM streaming read.
COMMITTED_CEILINGS = {"mfma_bf16_tflops": 2445.8, "mfma_fp8_tflops": 4921.3, "hbm_read_gbs": 7206.0,
                      "mfma_bf16_random_tflops": 1820.4, "mfma_fp8_random_tflops": 3839.0}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", dest="legs", action="store_true", default=True)
    ap.add_argument("--no-legs", dest="legs", action="store_false")
    ap.add_argument("--no-ceilings", action="store_true", help="use the committed ceilings, do not measure them")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    return ap.parse_args(argv)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dist(samples):
    """Summary of per-call durations in ms: count, mean, median, p10, p90, min, max."""
    import numpy as np
    x = np.asarray(samples, dtype=np.float64)
    if x.size == 0:
        return {"n": 0}
    return {"n": int(x.size), "mean_ms": float(x.mean()), "median_ms": float(np.median(x)),
            "p10_ms": float(np.percentile(x, 10)), "p90_ms": float(np.percentile(x, 90)), "min_ms": float(x.min()),
            "max_ms": float(x.max())}


def calibration_copy(torch, nbytes=1 << 30):
    """A plain elementwise copy kernel of known size (dst = -src over 1 GiB of float32: 1 GiB read,
    1 GiB written, larger than the last-level cache), run once before timing. Its FETCH_SIZE /
    WRITE_SIZE counters in a profiler run of this same command calibrate the byte counters of the
    attention kernels."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def kernel_sources_digest(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "roofline_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when the
    summary is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("kernels", {}).get(kernel)
    if not ent or ent.get("sources_sha256") != kernel_sources_digest(ent.get("sources", [])):
        return None
    return ent["hbm_bytes_per_launch"]


def ceilings(measure: bool):
    """MFMA and HBM ceilings of this GPU: measured now by the ceiling microbenchmarks (a child
    process), or the committed values when measuring is off or the executable is missing."""
    if measure:
        try:
            from roofline_attention_amd import ceilings as C
            m = C.measure(timeout=180.0)
            return {"source": "measured in this run (roofline_attention_amd/ceilings)",
                    **{k: float(m[k]) for k in COMMITTED_CEILINGS}}
        except (OSError, ValueError, KeyError, subprocess.SubprocessError) as e:
            log(f"[bench] ceilings not measured ({type(e).__name__}: {e}); using the committed values")
    return {"source": "committed measurement of the ceiling microbenchmarks on one MI355X", **COMMITTED_CEILINGS}


def warm_up(torch, fn, seconds=WARMUP_S, min_calls=3):
    """Untimed calls of fn() for at least `seconds` of wall time and at least `min_calls` calls:
    after the host-side input setup the GPU has idled and its clock ramps up again over the first
    tens of milliseconds of load."""
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_calls(torch, lib, fn, calls, between=None):
    """Three passes of `calls` calls of fn(), each ended by a synchronisation:
    1. back to back with the library timer off and no event between calls (skipped when `between`
       is given): host wall time and the device time between events at the loop's two ends;
    2. an event pair on the launch stream around each call, timer off: the per-call distribution
       (these events sit at call boundaries only, so a call's kernels run as they would untimed);
    3. the library timer on: every launch's duration from events recorded around it.
    `between`, if given, runs before each call outside the timer and outside the call's events (e.g.
    a cache flush). Returns a dict: wall_s and loop_ms (pass 1, or None), per_call (ms, pass 2),
    per_kernel ({kernel: [ms]}, pass 3)."""
    res = {"wall_s": None, "loop_ms": None}
    lib.timing_enable(False)
    if between is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(calls):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res["wall_s"] = time.perf_counter() - t0
        res["loop_ms"] = e0.elapsed_time(e1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    torch.cuda.synchronize()
    for a, b in ev:
        if between is not None:
            between()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    res["per_call"] = [a.elapsed_time(b) for a, b in ev]
    lib.timing_reset()
    lib.timing_enable(True)
    for _ in range(calls):
        if between is not None:
            lib.timing_enable(False)
            between()
            lib.timing_enable(True)
        fn()
    torch.cuda.synchronize()
    lib.timing_enable(False)
    res["per_kernel"] = lib.timing_samples()
    lib.timing_reset()
    return res


def time_graph(torch, fn, calls, replays=GRAPH_REPLAYS):
    """fn() captured `calls` times into one HIP graph (the library only enqueues kernels on the
    current stream), replayed `replays` times with an event pair around each replay: per-call device
    time without host launch cost, for launch-bound shapes. Returns per-replay ms / calls."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for a, b in ev:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    out = [a.elapsed_time(b) / calls for a, b in ev]
    del graph
    return out


def host_record():
    """CPU model, sockets, NUMA nodes and the CPUs this process may run on."""
    model, sockets = None, set()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name") and model is None:
                    model = line.split(":", 1)[1].strip()
                elif line.startswith("physical id"):
                    sockets.add(line.split(":", 1)[1].strip())
    except OSError:
        pass
    try:
        numa = len([n for n in os.listdir("/sys/devices/system/node") if n.startswith("node") and n[4:].isdigit()])
    except OSError:
        numa = None
    return {"cpu_model": model or platform.processor() or platform.machine(),
            "sockets": len(sockets) or None, "numa_nodes": numa,
            "affinity_cpus": len(os.sched_getaffinity(0)), "os_cpus": os.cpu_count()}


def cpu_baseline(w, target_s):
    """The fp64 oracle's forward+backward on whole heads of the same workload until ~target_s elapse."""
    from threadpoolctl import threadpool_info

    from oracle import attention as orc
    from roofline_attention_amd import inputs as I
    from roofline_attention_amd import ledger as L

    t = I.make_prefill(w, with_dout=True)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, elapsed = 0, 0.0
    while done < len(heads) and (elapsed < target_s or done == 0):
        b, h = heads[done]
        sl = (slice(b, b + 1), slice(h, h + 1))
        args = [I.to_f64(t[n][sl]) for n in ("q", "k", "v", "do")]
        t0 = time.perf_counter()
        orc.attention_bwd(*args, w.causal, w.scale)  # also computes O and LSE (the forward)
        elapsed += time.perf_counter() - t0
        done += 1
    flops = done * (L.fwd_flops(1, 1, w.N, w.d, w.causal) + L.bwd_flops(1, 1, w.N, w.d, w.causal))
    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] or [1])
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} (b,h) heads of the same workload, fp64 numpy forward+backward "
                  f"with explicit S, {elapsed:.2f} s wall; algorithmic FLOPs (causal halved) / time",
        "host": {**host_record(), "blas": sorted({p.get("internal_api", "?") for p in pools}),
                 "blas_threads": int(threads)},
    }


def rate_of(kind, amount, ms, ceil):
    """Algorithmic rate of `amount` FLOPs or bytes done in `ms`, with its fractions of the published
    peak and of the measured ceiling."""
    from roofline_attention_amd import ledger as L
    if kind in ("mfma", "mfma8"):
        r = amount / (ms * 1e-3) / 1e12
        fp8 = kind == "mfma8"
        out = {"tflops": r, "frac_of_peak": r / (L.PEAK_FP8_TFLOPS if fp8 else L.PEAK_BF16_TFLOPS),
               "frac_of_ceiling": r / ceil["mfma_fp8_tflops" if fp8 else "mfma_bf16_tflops"]}
        data = ceil.get("mfma_fp8_random_tflops" if fp8 else "mfma_bf16_random_tflops")
        if data:  # the same instruction's rate on operands like the kernel's
            out["frac_of_data_ceiling"] = r / data
        return out
    r = amount / (ms * 1e-3) / 1e9
    return {"gbs": r, "frac_of_peak": r / L.PEAK_HBM_GBS, "frac_of_ceiling": r / ceil["hbm_read_gbs"]}


def roofline_time(flops, peak_tflops, nbytes, ms):
    """The roofline time of one call, max(work / matrix peak, compulsory bytes / HBM peak), which of the
    two bounds it, and the measured time's fraction of it (1.0 = at the roofline)."""
    from roofline_attention_amd import ledger as L
    t_mfma = flops / (peak_tflops * 1e12) * 1e3
    t_hbm = nbytes / (L.PEAK_HBM_GBS * 1e9) * 1e3
    t = max(t_mfma, t_hbm)
    return {"bound": "mfma" if t_mfma >= t_hbm else "hbm", "mfma_ms": t_mfma, "hbm_ms": t_hbm,
            "compulsory_bytes": nbytes, "frac": t / ms}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (this library runs on a single "
              f"MI355X and has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    from roofline_attention_amd import binding as lib
    from roofline_attention_amd import inputs as I
    from roofline_attention_amd import ledger as L

    ceil = ceilings(not a.no_ceilings)
    log(f"[bench] ceilings: {ceil}")
    torch.cuda.set_device(0)
    calibration_copy(torch)
    w = I.WORKLOADS["fwdbwd_4k_causal"]
    log(f"[bench] inputs {w}")
    t = {k: x.cuda() for k, x in I.make_prefill(w, with_dout=True).items()}
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    ws = torch.empty(lib.bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")

    def step():
        lib.fwd(q, k, v, w.causal, w.scale, out=o, lse=lse)
        lib.bwd(q, k, v, o, do, lse, w.causal, w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    t_w = time.perf_counter()
    n_warm = warm_up(torch, step, seconds=WARMUP_S, min_calls=a.warmup)
    warm_s = time.perf_counter() - t_w
    log(f"[bench] warm-up {n_warm} steps in {warm_s:.2f} s; timing {a.steps} steps")
    tm = time_calls(torch, lib, step, a.steps)
    wall, per_kernel, per_step = tm["wall_s"], tm["per_kernel"], tm["per_call"]
    ms_per_step = wall / a.steps * 1e3
    step_flops = L.fwd_flops(w.B, w.H, w.N, w.d, w.causal) + L.bwd_flops(w.B, w.H, w.N, w.d, w.causal)
    value = step_flops / (wall / a.steps) / 1e12
    log(f"[bench] step {ms_per_step:.3f} ms -> {value:.1f} TFLOP/s")

    # Algorithmic work per launch of each kernel of the step. The backward's five products are
    # assigned where they are first computed: S, dP, dV, dK in the key-major kernel, dQ in the
    # query-major kernel (which also computes the rows' D from O and dO).
    Nsq = w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    work = {
        "fwd_bf16_d128_causal": ("mfma", 4.0 * Nsq),
        "bwd_dkdv_d128_causal": ("mfma", 8.0 * Nsq),
        "bwd_dq_d128_causal": ("mfma", 2.0 * Nsq),
    }
    kernels = {}
    for name, smp in per_kernel.items():
        kind, amount = work.get(name, (None, None))
        ent = {"launches": len(smp), **dist(smp)}
        if kind is not None:
            ent["avg_ms"] = ent["mean_ms"]
            ent.update(rate_of(kind, amount, ent["mean_ms"], ceil))
            ent["at_median"] = rate_of(kind, amount, ent["median_ms"], ceil)
        kernels[name] = ent
    dom = max(per_kernel, key=lambda n: sum(per_kernel[n]))
    kind, amount = work[dom]
    d = kernels[dom]
    roof = {"kernel": dom, "bound": "mfma", "achieved": d["tflops"], "peak": L.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": d["frac_of_peak"], "traffic": measured_traffic(dom),
            "ceiling": ceil["mfma_bf16_tflops"], "frac_of_ceiling": d["frac_of_ceiling"],
            "data_ceiling": ceil.get("mfma_bf16_random_tflops"), "frac_of_data_ceiling": d.get("frac_of_data_ceiling"),
            "avg_ms": d["mean_ms"], "median_ms": d["median_ms"], "p10_ms": d["p10_ms"], "p90_ms": d["p90_ms"],
            "min_ms": d["min_ms"], "algorithmic_per_launch": amount,
            "samples_ms": [round(x, 5) for x in per_kernel[dom]]}

    legs = {}
    if a.legs:
        del q, k, v, do, o, lse, dq, dk, dv, ws, t
        torch.cuda.empty_cache()
        legs = run_legs(torch, lib, I, L, ceil)

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, a.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "warmup_calls": n_warm,
        "warmup_s": warm_s,
        "ms_per_step": ms_per_step,
        "loop_device_ms_per_step": tm["loop_ms"] / a.steps,
        "step_device_ms": dist(per_step),
        "step_samples_ms": [round(x, 5) for x in per_step],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), per-(tensor,batch,head) numpy PCG64 streams, bf16 RNE)",
        "config": {"workload": "causal bf16 attention forward+backward B=2 H=16 N=4096 d=128 (fp32 grads)",
                   "global_batch": w.B, "heads": w.H, "seq_len": w.N, "head_dim": w.d, "causal": True,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "ceilings": ceil,
        "kernels": kernels,
        "legs": legs,
    }
    print(json.dumps(out), flush=True)


def leg_record(tm, calls, kind, amount, ceil, kernel=None):
    """One leg from time_calls' passes. The leg's time per call (avg_ms, and the rates) is the device
    time of the back-to-back loop divided by the calls (pass 1), or, for legs with work between
    calls, the mean of the per-call event pairs (pass 2). `kernels` holds each kernel's launch
    durations from the library timer (pass 3), whose events around every launch add a few
    microseconds to each."""
    ks = {n: dist(s) for n, s in tm["per_kernel"].items()}
    pc = dist(tm["per_call"])
    if tm["loop_ms"] is not None:
        mean_ms, med_ms, source = tm["loop_ms"] / calls, pc["median_ms"], "back-to-back loop"
    else:
        mean_ms, med_ms, source = pc["mean_ms"], pc["median_ms"], "per-call events"
    rec = {"avg_ms": mean_ms, "time_source": source, **rate_of(kind, amount, mean_ms, ceil),
           "at_median": rate_of(kind, amount, med_ms, ceil), "call_device_ms": pc, "kernels": ks,
           "kernels_sum_ms": sum(v["mean_ms"] for v in ks.values())}
    if tm["loop_ms"] is not None:
        rec["loop_ms_per_call"] = tm["loop_ms"] / calls
        rec["wall_ms_per_call"] = tm["wall_s"] / calls * 1e3
    if kernel is not None:
        rec["kernel"] = kernel
    return rec


def run_legs(torch, lib, I, L, ceil, calls=LEG_CALLS):
    """Extra legs: the 4k prefill forward (causal and not; bf16, then fp8 inputs), the 1k causal
    prefill, the step's forward+backward as one launch, the ragged prefill and its backward, GQA
    decode over a contiguous and over a paged cache (each cold and warm)."""
    legs = {}

    def timed(fn, between=None):
        warm_up(torch, (lambda: (between(), fn())) if between else fn)
        return time_calls(torch, lib, fn, calls, between)

    for name in ("prefill_4k_causal", "prefill_4k", "prefill_causal_1k"):
        w = I.WORKLOADS[name]
        t = {k: x.cuda() for k, x in I.make_prefill(w, with_dout=False).items()}
        o = torch.empty_like(t["q"])
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        def call():
            lib.fwd(t["q"], t["k"], t["v"], w.causal, w.scale, out=o, lse=lse)
        tm = timed(call)
        (kname,) = tm["per_kernel"]
        legs[name] = leg_record(tm, calls, "mfma", L.fwd_flops(w.B, w.H, w.N, w.d, w.causal), ceil, kname)
        legs[name]["roofline"] = roofline_time(L.fwd_flops(w.B, w.H, w.N, w.d, w.causal), L.PEAK_BF16_TFLOPS,
                                               L.fwd_bytes(w.B, w.H, w.H_kv, w.N, w.d, 2), legs[name]["avg_ms"])
        if name == "prefill_causal_1k":
            # a launch-bound call: the same calls replayed from a HIP graph, for comparison
            g = dist(time_graph(torch, call, calls))
            legs[name]["graph_replay"] = {"ms_per_call": g, **rate_of("mfma", L.fwd_flops(w.B, w.H, w.N, w.d, w.causal),
                                                                       g["mean_ms"], ceil)}
        log(f"[bench] leg {name}: {legs[name]['avg_ms']:.4f} ms ({legs[name]['time_source']}), "
            f"{legs[name]['tflops']:.1f} TFLOP/s, {legs[name]['roofline']['frac']:.3f} of its roofline "
            f"({legs[name]['roofline']['bound']}-bound)")
        del t, o, lse
        torch.cuda.empty_cache()

    # fp8 (E4M3) inputs: the same 4k prefill, priced against the fp8 matrix-core peak
    for name in ("prefill_4k_causal_fp8", "prefill_4k_fp8"):
        w = I.WORKLOADS[name]
        t8 = I.make_fp8_prefill(w)
        ds = t8.pop("descale")
        t = {k: x.cuda() for k, x in t8.items()}
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        tm = timed(lambda: lib.fwd_fp8(t["q"], t["k"], t["v"], ds, w.causal, w.scale, out=o, lse=lse))
        (kname,) = tm["per_kernel"]
        legs[name] = leg_record(tm, calls, "mfma8", L.fwd_flops(w.B, w.H, w.N, w.d, w.causal), ceil, kname)
        legs[name]["peak_tflops"] = L.PEAK_FP8_TFLOPS
        log(f"[bench] leg {name}: {legs[name]['avg_ms']:.4f} ms, {legs[name]['tflops']:.1f} TFLOP/s "
            f"({legs[name]['frac_of_peak']:.3f} of fp8 peak)")
        del t, t8, o, lse
        torch.cuda.empty_cache()

    # The same forward+backward as the step, as one cooperative launch (attn_fwd_bwd)
    w = I.WORKLOADS["fwdbwd_4k_causal"]
    t = {k: x.cuda() for k, x in I.make_prefill(w, with_dout=True).items()}
    outs = dict(o=torch.empty_like(t["q"]), lse=torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda"),
                dq=torch.empty(t["q"].shape, dtype=torch.float32, device="cuda"))
    outs["dk"], outs["dv"] = torch.empty_like(outs["dq"]), torch.empty_like(outs["dq"])
    wsf = torch.empty(lib.fwd_bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
    tm = timed(lambda: lib.fwd_bwd(t["q"], t["k"], t["v"], t["do"], w.causal, w.scale, workspace=wsf, **outs))
    (kname,) = tm["per_kernel"]
    fl = L.fwd_flops(w.B, w.H, w.N, w.d, w.causal) + L.bwd_flops(w.B, w.H, w.N, w.d, w.causal)
    legs["fwdbwd_fused"] = leg_record(tm, calls, "mfma", fl, ceil, kname)
    legs["fwdbwd_fused"]["launches_per_call"] = 1
    log(f"[bench] leg fwdbwd_fused: {legs['fwdbwd_fused']['avg_ms']:.3f} ms, {legs['fwdbwd_fused']['tflops']:.1f} "
        f"TFLOP/s (one launch)")
    del t, outs, wsf
    torch.cuda.empty_cache()

    w = I.WORKLOADS["prefill_varlen"]
    t = I.make_varlen(w, with_dout=True)
    lengths = t["lengths"]
    cu = t["cu_seqlens"].cuda()
    t = {k: t[k].cuda() for k in ("q", "k", "v", "do")}
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.H, t["q"].shape[0]), dtype=torch.float32, device="cuda")
    max_len = int(lengths.max())
    tm = timed(lambda: lib.fwd_varlen(t["q"], t["k"], t["v"], cu, max_len, w.causal, w.scale, out=o, lse=lse))
    (kname,) = tm["per_kernel"]
    legs["prefill_varlen"] = leg_record(tm, calls, "mfma", L.varlen_fwd_flops(w.H, w.d, lengths, w.causal), ceil,
                                        kname)
    legs["prefill_varlen"].update(tokens=int(lengths.sum()), sequences=int(len(lengths)), max_len=max_len)
    log(f"[bench] leg prefill_varlen: {legs['prefill_varlen']['avg_ms']:.3f} ms, "
        f"{legs['prefill_varlen']['tflops']:.1f} TFLOP/s ({int(lengths.sum())} tokens in {len(lengths)} sequences)")

    # The backward of the same ragged batch (attn_bwd_varlen: dQ kernel, then dK/dV kernel)
    f32 = dict(dtype=torch.float32, device="cuda")
    g = dict(dq=torch.empty(t["q"].shape, **f32), dk=torch.empty(t["k"].shape, **f32),
             dv=torch.empty(t["v"].shape, **f32))
    wsv = torch.empty(lib.bwd_varlen_workspace_size(t["q"].shape[0], w.H, w.d), dtype=torch.uint8, device="cuda")
    tm = timed(lambda: lib.bwd_varlen(t["q"], t["k"], t["v"], o, t["do"], lse, cu, max_len, w.causal, w.scale,
                                      workspace=wsv, **g))
    fl = sum(L.bwd_flops(1, w.H, int(n), w.d, w.causal) for n in lengths)
    legs["prefill_varlen_bwd"] = leg_record(tm, calls, "mfma", fl, ceil)
    log(f"[bench] leg prefill_varlen_bwd: {legs['prefill_varlen_bwd']['avg_ms']:.3f} ms, "
        f"{legs['prefill_varlen_bwd']['tflops']:.1f} TFLOP/s (two kernels)")
    del t, o, lse, cu, g, wsv
    torch.cuda.empty_cache()

    w = I.WORKLOADS["decode_gqa"]
    dense = I.make_decode(w)
    lens = dense["kv_len"].numpy().tolist()
    nbytes = L.decode_bytes(w.H, w.H_kv, w.d, 2, lens)
    # Read (not written) before each cold call to evict the cache: a written buffer would leave dirty
    # lines whose write-back then lands inside the timed kernel.
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB, above the 256 MB last-level cache
    o = torch.empty((w.B, w.H, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    wsd = torch.zeros(lib.decode_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")

    def decode_leg(fn, name, extra):
        # cold (primary): every byte comes from HBM; warm: back-to-back calls, part of the 1.06 GB may
        # still sit in the 256 MB last-level cache
        tm = timed(fn, between=lambda: flush.sum())
        rec = leg_record(tm, calls, "hbm", nbytes, ceil)
        split = [n for n in tm["per_kernel"] if "split" in n][0]
        rec.update(compulsory_bytes=nbytes, cache="cold (1 GiB buffer read before each call, outside the timed "
                                                   "kernels and the call's events)",
                   split_kernel=rate_of("hbm", nbytes, rec["kernels"][split]["mean_ms"], ceil),
                   tflops=L.decode_flops(w.H, w.d, lens) / (rec["avg_ms"] * 1e-3) / 1e12, **extra)
        warm = leg_record(timed(fn), calls, "hbm", nbytes, ceil)
        rec["warm"] = {"avg_ms": warm["avg_ms"], "gbs": warm["gbs"], "frac_of_peak": warm["frac_of_peak"],
                       "kernels": warm["kernels"], "call_device_ms": warm["call_device_ms"]}
        legs[name] = rec
        log(f"[bench] leg {name}: {rec['avg_ms']:.4f} ms over {len(tm['per_kernel'])} kernel(s), {rec['gbs']:.0f} GB/s "
            f"({rec['frac_of_peak']:.3f} of 8 TB/s whole call; split kernel {rec['split_kernel']['gbs']:.0f} GB/s); "
            f"warm {rec['warm']['gbs']:.0f} GB/s")

    t = {k: x.cuda() for k, x in dense.items()}
    decode_leg(lambda: lib.decode(t["q"], t["k"], t["v"], t["kv_len"], w.scale, out=o, lse=lse, workspace=wsd),
               "decode_gqa", {})
    del t
    paged = I.make_decode_paged(w, 64, dense=dense)
    del dense
    tp = {k: x.cuda() for k, x in paged.items()}
    decode_leg(lambda: lib.decode_paged(tp["q"], tp["k_pages"], tp["v_pages"], tp["block_table"], tp["kv_len"],
                                        w.scale, out=o, lse=lse, workspace=wsd),
               "decode_gqa_paged", {"page_size": 64, "pages": int(paged["k_pages"].shape[0]),
                                    "placement": "seeded shuffle"})
    return legs


if __name__ == "__main__":
    main()
