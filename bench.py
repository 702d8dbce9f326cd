"""Benchmark of the attention hot path on one MI355X.

A step is one forward + backward pass (attn_fwd then attn_bwd, all forward and backward kernels)
of causal bf16 attention over the [B=2, H=16, N=4096, d=128] synthetic batch, inputs resident in
HBM before timing starts. The decode kernels and the two 4k prefill forwards are timed as extra
legs in the same run and reported beside the step. Kernel durations come from HIP events that
the library records on its launch stream around every kernel while its timer is enabled.

Output: one JSON line on stdout (rank 0), with the roofline of the dominant kernel and the fp64
CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--legs/--no-legs]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd/bwd TFLOP/s and decode HBM GB/s, % of MI355X roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", dest="legs", action="store_true", default=True)
    ap.add_argument("--no-legs", dest="legs", action="store_false")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_stats(lib, before=None):
    rec = lib.timing_read()
    return {k: {"launches": n, "avg_ms": ms / n if n else None, "total_ms": ms} for k, (n, ms) in rec.items()}


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


def warm_up(torch, fn, seconds=0.2, min_calls=3):
    """Untimed calls of fn() for at least `seconds` of wall time: after the host-side input setup
    the GPU has idled and its clock ramps up again over the first tens of milliseconds of load."""
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_region(torch, lib, fn, steps):
    """Runs fn() `steps` times between synchronisations; returns (wall seconds, kernel stats)."""
    lib.timing_reset()
    torch.cuda.synchronize()
    lib.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lib.timing_enable(False)
    stats = kernel_stats(lib)
    lib.timing_reset()
    return t1 - t0, stats


def cpu_baseline(w, target_s):
    """The fp64 oracle's forward+backward on whole heads of the same workload until ~target_s elapse."""
    import numpy as np
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
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} (b,h) heads of the same workload, fp64 numpy forward+backward "
                  f"with explicit S, {elapsed:.2f} s wall; algorithmic FLOPs (causal halved) / time",
        "host": platform.processor() or platform.machine(),
    }


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

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {a.warmup} done; timing {a.steps} steps")
    wall, stats = time_region(torch, lib, step, a.steps)
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
    for name, st in stats.items():
        kind, amount = work.get(name, (None, None))
        ent = dict(st)
        if kind == "mfma" and st["avg_ms"]:
            ent["tflops"] = amount / (st["avg_ms"] * 1e-3) / 1e12
            ent["frac_of_peak"] = ent["tflops"] / L.PEAK_BF16_TFLOPS
        elif kind == "hbm" and st["avg_ms"]:
            ent["gbs"] = amount / (st["avg_ms"] * 1e-3) / 1e9
            ent["frac_of_peak"] = ent["gbs"] / L.PEAK_HBM_GBS
        kernels[name] = ent
    dom = max(stats, key=lambda n: stats[n]["total_ms"])
    kind, amount = work[dom]
    avg_s = stats[dom]["avg_ms"] * 1e-3
    if kind == "mfma":
        roof = {"kernel": dom, "bound": "mfma", "achieved": amount / avg_s / 1e12, "peak": L.PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": amount / avg_s / 1e9, "peak": L.PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom)
    roof["avg_ms"] = stats[dom]["avg_ms"]
    roof["algorithmic_per_launch"] = amount

    legs = {}
    if a.legs:
        del q, k, v, do, o, lse, dq, dk, dv, ws, t
        torch.cuda.empty_cache()
        legs = run_legs(torch, lib, I, L)

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
        "ms_per_step": ms_per_step,
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
        "kernels": kernels,
        "legs": legs,
    }
    print(json.dumps(out), flush=True)


def run_legs(torch, lib, I, L, reps=20):
    """Extra legs: the 4k prefill forward (causal and not; bf16, then fp8 inputs), the 1k causal
    prefill, the step's forward+backward as one launch, the ragged prefill and its backward, GQA
    decode over a contiguous and over a paged cache."""
    legs = {}
    for name in ("prefill_4k_causal", "prefill_4k", "prefill_causal_1k"):
        w = I.WORKLOADS[name]
        t = {k: x.cuda() for k, x in I.make_prefill(w, with_dout=False).items()}
        o = torch.empty_like(t["q"])
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        fn = lambda: lib.fwd(t["q"], t["k"], t["v"], w.causal, w.scale, out=o, lse=lse)  # noqa: E731
        warm_up(torch, fn)
        wall, stats = time_region(torch, lib, fn, reps)
        (kname, st), = stats.items()
        fl = L.fwd_flops(w.B, w.H, w.N, w.d, w.causal)
        legs[name] = {"kernel": kname, "avg_ms": st["avg_ms"], "tflops": fl / (st["avg_ms"] * 1e-3) / 1e12,
                      "frac_of_peak": fl / (st["avg_ms"] * 1e-3) / 1e12 / L.PEAK_BF16_TFLOPS,
                      "wall_ms_per_call": wall / reps * 1e3}
        log(f"[bench] leg {name}: {legs[name]['avg_ms']:.3f} ms, {legs[name]['tflops']:.1f} TFLOP/s")
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
        fn = lambda: lib.fwd_fp8(t["q"], t["k"], t["v"], ds, w.causal, w.scale, out=o, lse=lse)  # noqa: E731
        warm_up(torch, fn)
        wall, stats = time_region(torch, lib, fn, reps)
        (kname, st), = stats.items()
        fl = L.fwd_flops(w.B, w.H, w.N, w.d, w.causal)
        tf = fl / (st["avg_ms"] * 1e-3) / 1e12
        legs[name] = {"kernel": kname, "avg_ms": st["avg_ms"], "tflops": tf, "frac_of_peak": tf / L.PEAK_FP8_TFLOPS,
                      "peak_tflops": L.PEAK_FP8_TFLOPS, "wall_ms_per_call": wall / reps * 1e3}
        log(f"[bench] leg {name}: {st['avg_ms']:.3f} ms, {tf:.1f} TFLOP/s ({tf / L.PEAK_FP8_TFLOPS:.3f} of fp8 peak)")
        del t, t8, o, lse
        torch.cuda.empty_cache()

    # The same forward+backward as the step, as one cooperative launch (attn_fwd_bwd)
    w = I.WORKLOADS["fwdbwd_4k_causal"]
    t = {k: x.cuda() for k, x in I.make_prefill(w, with_dout=True).items()}
    outs = dict(o=torch.empty_like(t["q"]), lse=torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda"),
                dq=torch.empty(t["q"].shape, dtype=torch.float32, device="cuda"))
    outs["dk"], outs["dv"] = torch.empty_like(outs["dq"]), torch.empty_like(outs["dq"])
    wsf = torch.empty(lib.fwd_bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
    fn = lambda: lib.fwd_bwd(t["q"], t["k"], t["v"], t["do"], w.causal, w.scale, workspace=wsf, **outs)  # noqa
    warm_up(torch, fn)
    wall, stats = time_region(torch, lib, fn, reps)
    (kname, st), = stats.items()
    fl = L.fwd_flops(w.B, w.H, w.N, w.d, w.causal) + L.bwd_flops(w.B, w.H, w.N, w.d, w.causal)
    tf = fl / (st["avg_ms"] * 1e-3) / 1e12
    legs["fwdbwd_fused"] = {"kernel": kname, "avg_ms": st["avg_ms"], "tflops": tf, "frac_of_peak": tf / L.PEAK_BF16_TFLOPS,
                            "wall_ms_per_call": wall / reps * 1e3, "launches_per_call": 1}
    log(f"[bench] leg fwdbwd_fused: {st['avg_ms']:.3f} ms, {tf:.1f} TFLOP/s (one launch)")
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
    fn = lambda: lib.fwd_varlen(t["q"], t["k"], t["v"], cu, max_len, w.causal, w.scale, out=o, lse=lse)  # noqa
    warm_up(torch, fn)
    wall, stats = time_region(torch, lib, fn, reps)
    (kname, st), = stats.items()
    fl = L.varlen_fwd_flops(w.H, w.d, lengths, w.causal)
    legs["prefill_varlen"] = {"kernel": kname, "avg_ms": st["avg_ms"], "tflops": fl / (st["avg_ms"] * 1e-3) / 1e12,
                              "frac_of_peak": fl / (st["avg_ms"] * 1e-3) / 1e12 / L.PEAK_BF16_TFLOPS,
                              "wall_ms_per_call": wall / reps * 1e3, "tokens": int(lengths.sum()),
                              "sequences": int(len(lengths)), "max_len": max_len}
    log(f"[bench] leg prefill_varlen: {st['avg_ms']:.3f} ms, {legs['prefill_varlen']['tflops']:.1f} TFLOP/s "
        f"({int(lengths.sum())} tokens in {len(lengths)} sequences)")

    # The backward of the same ragged batch (attn_bwd_varlen: dQ kernel, then dK/dV kernel)
    f32 = dict(dtype=torch.float32, device="cuda")
    g = dict(dq=torch.empty(t["q"].shape, **f32), dk=torch.empty(t["k"].shape, **f32),
             dv=torch.empty(t["v"].shape, **f32))
    wsv = torch.empty(lib.bwd_varlen_workspace_size(t["q"].shape[0], w.H, w.d), dtype=torch.uint8, device="cuda")
    fn = lambda: lib.bwd_varlen(t["q"], t["k"], t["v"], o, t["do"], lse, cu, max_len, w.causal, w.scale,  # noqa
                                workspace=wsv, **g)
    warm_up(torch, fn)
    wall, stats = time_region(torch, lib, fn, reps)
    ms = sum(st["avg_ms"] for st in stats.values())
    fl = sum(L.bwd_flops(1, w.H, int(n), w.d, w.causal) for n in lengths)
    tf = fl / (ms * 1e-3) / 1e12
    legs["prefill_varlen_bwd"] = {"kernels": {k: st["avg_ms"] for k, st in stats.items()}, "avg_ms": ms, "tflops": tf,
                                  "frac_of_peak": tf / L.PEAK_BF16_TFLOPS, "wall_ms_per_call": wall / reps * 1e3}
    log(f"[bench] leg prefill_varlen_bwd: {ms:.3f} ms, {tf:.1f} TFLOP/s (two kernels)")
    del t, o, lse, cu, g, wsv
    torch.cuda.empty_cache()

    w = I.WORKLOADS["decode_gqa"]
    dense = I.make_decode(w)
    lens = dense["kv_len"].numpy().tolist()
    nbytes = L.decode_bytes(w.H, w.H_kv, w.d, 2, lens)
    # Read (not written) before each call to evict the cache: a written buffer would leave dirty
    # lines whose write-back then lands inside the timed kernel.
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB, above the 256 MB last-level cache
    o = torch.empty((w.B, w.H, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    wsd = torch.empty(lib.decode_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")

    def cold_decode(fn, name, split_prefix, extra):
        warm_up(torch, lambda: (flush.sum(), fn()))
        # cold: the cache flush runs outside the timed kernels
        lib.timing_reset()
        lib.timing_enable(True)
        for _ in range(reps):
            lib.timing_enable(False)
            flush.sum()
            lib.timing_enable(True)
            fn()
        torch.cuda.synchronize()
        lib.timing_enable(False)
        stats = kernel_stats(lib)
        lib.timing_reset()
        total_ms = sum(s["avg_ms"] for s in stats.values())
        split = [n for n in stats if n.startswith(split_prefix)][0]
        legs[name] = {
            "kernels": {n: s["avg_ms"] for n, s in stats.items()},
            "compulsory_bytes": nbytes,
            "gbs_split_kernel": nbytes / (stats[split]["avg_ms"] * 1e-3) / 1e9,
            "gbs_both_kernels": nbytes / (total_ms * 1e-3) / 1e9,
            "frac_of_peak_split": nbytes / (stats[split]["avg_ms"] * 1e-3) / 1e9 / L.PEAK_HBM_GBS,
            "cache": "cold (1 GiB buffer read before each call, outside the timed kernels)",
            "tflops": L.decode_flops(w.H, w.d, lens) / (total_ms * 1e-3) / 1e12,
            **extra,
        }
        log(f"[bench] leg {name}: {total_ms:.3f} ms, {legs[name]['gbs_both_kernels']:.0f} GB/s")

    t = {k: x.cuda() for k, x in dense.items()}
    cold_decode(lambda: lib.decode(t["q"], t["k"], t["v"], t["kv_len"], w.scale, out=o, lse=lse, workspace=wsd),
                "decode_gqa", "decode_split", {})
    del t
    paged = I.make_decode_paged(w, 64, dense=dense)
    del dense
    tp = {k: x.cuda() for k, x in paged.items()}
    cold_decode(lambda: lib.decode_paged(tp["q"], tp["k_pages"], tp["v_pages"], tp["block_table"], tp["kv_len"],
                                         w.scale, out=o, lse=lse, workspace=wsd),
                "decode_gqa_paged", "decode_paged_split",
                {"page_size": 64, "pages": int(paged["k_pages"].shape[0]), "placement": "seeded shuffle"})
    return legs


if __name__ == "__main__":
    main()
