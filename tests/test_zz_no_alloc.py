"""attn_decode_noalloc (decode on the library's fixed per-GPU scratch, for callers that cannot
allocate) against attn_decode with a caller workspace: the same kernels on the same inputs, so the
outputs must agree bit for bit. Two calls in a row, the second on a smaller input, so the second
runs on scratch that holds the first call's records; plus the rejection of shapes beyond the
scratch (before any device work) and a check of the first call against the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import attention as orc
from roofline_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
SCRATCH = 16 << 20


def p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def call_noalloc(raw, t, w, o, lse):
    B, H, d = t["q"].shape
    return raw.attn_decode_noalloc(p(t["q"]), p(t["k"]), p(t["v"]), p(o), p(lse), p(t["kv_len"]), B, H, w.H_kv, w.N,
                                   d, 0, w.scale, 1, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def call_decode(raw, t, w, o, lse):
    B, H, d = t["q"].shape
    ws = torch.empty(raw.attn_decode_workspace_size(B, H, w.N, d), dtype=torch.uint8, device="cuda")
    return raw.attn_decode(p(t["q"]), p(t["k"]), p(t["v"]), p(o), p(lse), p(t["kv_len"]), B, H, w.H_kv, w.N, d, 0,
                           w.scale, 1, p(ws), ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def case(B, H, H_kv, N, d, seed, lens):
    w = I.Workload("noalloc", "decode", B, H, H_kv, N, d, "bf16", False, seed=seed, kv_lo=1, kv_hi=N)
    t = I.make_decode(w, nan_pad=False)
    t["kv_len"] = torch.tensor(lens, dtype=torch.int32)
    for b, n in enumerate(lens):  # rows past a sequence's length must never be read
        t["k"][b, :, n:] = float("nan")
        t["v"][b, :, n:] = float("nan")
    return w, t


def test_noalloc_matches_decode_on_two_calls_the_second_smaller(lib):
    raw = lib.raw()
    # first: the headline decode workload (64 sequences, 32/8 heads, d = 128, 512..8192 keys), 8.6 MB
    # of split records; second: a smaller batch with other group size, d and lengths
    w1 = I.WORKLOADS["decode_gqa"]
    t1 = I.make_decode(w1)
    w2, t2 = case(5, 12, 4, 3000, 64, seed=41, lens=[3000, 1, 1024, 1025, 2047])
    assert raw.attn_decode_workspace_size(w1.B, w1.H, w1.N, w1.d) <= SCRATCH
    results = []
    for w, t in ((w1, t1), (w2, t2)):
        g = {k: x.cuda() for k, x in t.items()}
        B, H, d = g["q"].shape
        o_n, o_d = torch.empty_like(g["q"]), torch.empty_like(g["q"])
        l_n = torch.empty((B, H), dtype=torch.float32, device="cuda")
        l_d = torch.empty_like(l_n)
        assert call_noalloc(raw, g, w, o_n, l_n) == 0, raw.attn_last_error()
        assert call_decode(raw, g, w, o_d, l_d) == 0, raw.attn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(o_n, o_d) and torch.equal(l_n, l_d)
        assert torch.isfinite(o_n.float()).all()
        results.append((w, t, o_n.cpu(), l_n.cpu()))
    # the second (smaller) call against the oracle as well
    w, t, o, lse = results[1]
    q = I.to_f64(t["q"])
    for b, n in enumerate(t["kv_len"].tolist()):
        ro, rl = orc.attention_decode(q[b:b + 1], I.to_f64(t["k"][b:b + 1, :, :n]), I.to_f64(t["v"][b:b + 1, :, :n]),
                                      np.array([n]), w.scale)
        assert float(np.max(np.abs(I.to_f64(o[b:b + 1]) - ro))) <= TOL_BF16
        assert float(np.max(np.abs(I.to_f64(lse[b:b + 1]) - rl))) <= TOL_BF16


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    raw = lib.raw()
    # 64 x 32 heads x 17 record slots (16k keys) x 132 floats = 18.4 MB of records > 16 MiB: rejected
    # before any device work (the pointers are never dereferenced)
    B, H, H_kv, N, d = 64, 32, 8, 16384, 128
    assert raw.attn_decode_workspace_size(B, H, N, d) > SCRATCH
    fake = [ctypes.c_void_p((1 << 40) + i * (1 << 34)) for i in range(6)]
    st = raw.attn_decode_noalloc(*fake, B, H, H_kv, N, d, 0, 0.088, 1, None)
    assert st == 3 and b"scratch" in raw.attn_last_error()  # ATTN_ERR_WORKSPACE
    # the binding reports it as an error too
    # 64 query heads over 1M cache rows at d = 64: 64 x 1025 record slots x 68 floats = 17.8 MB of records
    assert raw.attn_decode_workspace_size(1, 64, 1 << 20, 64) > SCRATCH
    q = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 8, 1 << 20, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.AttnError):
        lib.decode_noalloc(q, kc, kc, torch.tensor([5], dtype=torch.int32, device="cuda"))
