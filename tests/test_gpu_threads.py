"""Concurrent calls from several host threads, each on its own stream and buffers.

Runs in a fresh child process so that the threads also race on each kernel's first launch (where
the library raises the kernel's dynamic-LDS limit on the device). Every thread's results must equal
those of the same calls made one after another.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, threading
sys.path.insert(0, sys.argv[1])
import torch
from roofline_attention_amd import binding as lib, inputs as I

def job(i, causal, out):
    w = I.Workload(f"thr{i}", "fwdbwd", 1, 4, 2, 320 + 64 * i, 128, "bf16", causal, seed=40 + i)
    t = {k: x.cuda() for k, x in I.make_prefill(w, with_dout=True).items()}
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = lib.fwd(t["q"], t["k"], t["v"], causal, w.scale)
        g = lib.bwd(t["q"], t["k"], t["v"], o, t["do"], lse, causal, w.scale)
    s.synchronize()
    out[i] = (t, w, [x.cpu() for x in (o, lse, *g)])

results = {}
threads = [threading.Thread(target=job, args=(i, i % 2 == 0, results)) for i in range(4)]
for th in threads: th.start()
for th in threads: th.join()
assert len(results) == 4, "a thread failed"
for i, (t, w, got) in sorted(results.items()):
    causal = i % 2 == 0
    o, lse = lib.fwd(t["q"], t["k"], t["v"], causal, w.scale)
    g = lib.bwd(t["q"], t["k"], t["v"], o, t["do"], lse, causal, w.scale)
    torch.cuda.synchronize()
    ref = [x.cpu() for x in (o, lse, *g)]
    assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"thread {i} differs from the serial calls"
print("threads ok")
"""


def test_concurrent_threads_match_serial_calls():
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "threads ok" in r.stdout
