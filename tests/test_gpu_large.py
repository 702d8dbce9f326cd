"""Tensors past 4 GiB: every entry point addresses its inputs and outputs with 64-bit offsets.

Each case lays out at least one tensor larger than 2^32 bytes and checks the heads, sequences or
pages that sit past that offset (and a few before it) against the fp64 oracle, to the same
tolerances as the other parity tests. Inputs are seeded normal samples drawn on the GPU by torch
(chunk by chunk, to bound the temporaries); the checked slices are copied back for the oracle.
Cache rows and pages that a case must not read are left uninitialised, so reading them would put
arbitrary values, NaNs included, into the checked outputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as orc
from roofline_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
GIB = 1 << 30


def f64(t):
    return I.to_f64(t)


def max_err(gpu, ref):
    return float(np.max(np.abs(f64(gpu) - ref)))


def fill_normal(t: torch.Tensor, seed: int, factor: float = 1.0, chunk_rows: int = 4096):
    """Fills t (first dimension in chunks) with seeded N(0,1) * factor, rounded to t's dtype."""
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    for i in range(0, t.shape[0], chunk_rows):
        part = t[i:i + chunk_rows]
        x = torch.randn(part.shape, generator=g, device=t.device, dtype=torch.float32)
        if factor != 1.0:
            x *= factor
        part.copy_(x.to(t.dtype))
        del x


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_and_bwd_past_4gib(lib, causal):
    # [B, 2, 256, 128] bf16: 4.25 GiB per input, 8.5 GiB per fp32 gradient (B, H <= 65535).
    B, H, N, d = 34816, 2, 256, 128
    assert B * H * N * d * 2 > 4 * GIB
    scale = 1.0 / math.sqrt(d)
    print(f"large fwd+bwd causal={causal}: allocating", flush=True)
    q, k, v, do = (torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    for i, t in enumerate((q, k, v, do)):
        fill_normal(t, 100 + i, 0.5 if i < 2 else 1.0)
    o, lse = lib.fwd(q, k, v, causal, scale)
    dq, dk, dv = lib.bwd(q, k, v, o, do, lse, causal, scale)
    torch.cuda.synchronize()
    for b in (0, B // 2, B - 2, B - 1):  # the last heads start past 4 GiB (inputs) and 8 GiB (grads)
        sl = slice(b, b + 1)
        rdq, rdk, rdv, ro, rl = orc.attention_bwd(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]), causal, scale)
        assert max_err(o[sl], ro) <= TOL_BF16, b
        assert float(np.max(np.abs(lse[sl].cpu().numpy() - rl))) <= TOL_BF16, b
        for got, ref in ((dq, rdq), (dk, rdk), (dv, rdv)):
            assert max_err(got[sl], ref) <= TOL_BF16, b
    del q, k, v, do, o, lse, dq, dk, dv
    release()


def test_fused_fwd_bwd_past_4gib(lib):
    B, H, N, d = 34816, 2, 256, 128
    scale = 1.0 / math.sqrt(d)
    print("large fused fwd+bwd: allocating", flush=True)
    q, k, v, do = (torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    for i, t in enumerate((q, k, v, do)):
        fill_normal(t, 110 + i)
    o, lse, dq, dk, dv = lib.fwd_bwd(q, k, v, do, True, scale)
    torch.cuda.synchronize()
    for b in (1, B - 1):
        sl = slice(b, b + 1)
        rdq, rdk, rdv, ro, rl = orc.attention_bwd(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]), True, scale)
        assert max_err(o[sl], ro) <= TOL_BF16, b
        assert float(np.max(np.abs(lse[sl].cpu().numpy() - rl))) <= TOL_BF16, b
        for got, ref in ((dq, rdq), (dk, rdk), (dv, rdv)):
            assert max_err(got[sl], ref) <= TOL_BF16, b
    del q, k, v, do, o, lse, dq, dk, dv
    release()


def test_fp8_fwd_past_4gib(lib):
    # [B, 4, 256, 128] E4M3 codes: 4.25 GiB per input; O (bf16) 8.5 GiB.
    B, H, N, d = 34816, 4, 256, 128
    assert B * H * N * d > 4 * GIB
    scale = 1.0 / math.sqrt(d)
    print("large fp8 fwd: allocating", flush=True)
    codes = []
    for i in range(3):
        t = torch.empty((B, H, N, d), dtype=torch.float8_e4m3fn, device="cuda")
        # N(0,1) * 0.5 (q, k) or N(0,1) (v) stays far inside E4M3's range: descale 1.
        fill_normal(t, 120 + i, 0.5 if i < 2 else 1.0)
        codes.append(t.view(torch.uint8))
    descale = (1.0, 1.0, 1.0)
    o, lse = lib.fwd_fp8(codes[0], codes[1], codes[2], descale, True, scale)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        sl = slice(b, b + 1)
        ro, rl = orc.attention_fwd_fp8(*(c[sl].cpu().numpy() for c in codes), descale, True, scale)
        # The fp8 forward's own error model is tested at length elsewhere; a loose absolute bound
        # separates correct addressing (errors of order 2^-4 at most) from reading wrong rows.
        assert max_err(o[sl], ro) <= 0.1, b
        assert float(np.max(np.abs(lse[sl].cpu().numpy() - rl))) <= 0.05, b
    del codes, o, lse
    release()


def test_varlen_fwd_past_4gib(lib):
    # Packed [T, 1, 128] bf16 rows with T > 2^24: 4.25+ GiB per input.
    H, d = 1, 128
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([130, 0])))
    lens = g.integers(256, 768, size=34000, endpoint=True)
    lens[0], lens[-1] = 1, 768
    T = int(lens.sum())
    while T * H * d * 2 <= 4 * GIB + (1 << 20):
        lens = np.concatenate([lens, [384]])
        T = int(lens.sum())
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    scale = 1.0 / math.sqrt(d)
    print(f"large varlen fwd: T={T}, B={len(lens)}", flush=True)
    q, k, v = (torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    for i, t in enumerate((q, k, v)):
        fill_normal(t, 140 + i, 0.5 if i < 2 else 1.0, chunk_rows=1 << 20)
    o, lse = lib.fwd_varlen(q, k, v, torch.from_numpy(cu).cuda(), int(lens.max()), True, scale)
    torch.cuda.synchronize()
    for s in (0, len(lens) // 2, len(lens) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        view = lambda t: t[a:e].permute(1, 0, 2).unsqueeze(0)  # [1, H, n, d]
        ro, rl = orc.attention_fwd(f64(view(q)), f64(view(k)), f64(view(v)), True, scale)
        assert max_err(view(o), ro) <= TOL_BF16, s
        assert float(np.max(np.abs(lse[:, a:e].cpu().numpy() - rl[0]))) <= TOL_BF16, s
    del q, k, v, o, lse
    release()


def test_varlen_bwd_past_4gib(lib):
    # The ragged backward over packed [T, 1, 128] rows, T > 2^24: bf16 inputs past 4 GiB, fp32
    # gradients past 8 GiB.
    H, d = 1, 128
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([180, 0])))
    lens = g.integers(256, 768, size=34000, endpoint=True)
    lens[0], lens[-1] = 5, 700
    T = int(lens.sum())
    while T * H * d * 2 <= 4 * GIB + (1 << 20):
        lens = np.concatenate([lens, [384]])
        T = int(lens.sum())
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    scale = 1.0 / math.sqrt(d)
    print(f"large varlen bwd: T={T}, B={len(lens)}", flush=True)
    q, k, v, do = (torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    for i, t in enumerate((q, k, v, do)):
        fill_normal(t, 190 + i, 0.5 if i < 2 else 1.0, chunk_rows=1 << 20)
    cud = torch.from_numpy(cu).cuda()
    ml = int(lens.max())
    o, lse = lib.fwd_varlen(q, k, v, cud, ml, True, scale)
    dq, dk, dv = lib.bwd_varlen(q, k, v, o, do, lse, cud, ml, True, scale)
    torch.cuda.synchronize()
    for s in (0, len(lens) // 2, len(lens) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        rdq, rdk, rdv, _, _ = orc.attention_bwd_varlen(f64(q[a:e]), f64(k[a:e]), f64(v[a:e]), f64(do[a:e]),
                                                       [0, e - a], True, scale)
        for got, ref in ((dq, rdq), (dk, rdk), (dv, rdv)):
            assert max_err(got[a:e], ref) <= TOL_BF16, s
    del q, k, v, do, o, lse, dq, dk, dv, cud
    release()


def test_decode_cache_past_4gib(lib):
    # [5, 8, 2^19, 128] bf16 caches: 5 GiB each; sequence 4's rows start at 4 GiB.
    B, H, H_kv, N_cap, d = 5, 32, 8, 1 << 19, 128
    assert B * H_kv * N_cap * d * 2 > 4 * GIB
    kv_len = [700, 2049, 1, 4129, 3000]
    scale = 1.0 / math.sqrt(d)
    print("large decode: allocating", flush=True)
    kc = torch.empty((B, H_kv, N_cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    for b, n in enumerate(kv_len):  # rows past kv_len stay uninitialised
        for hk in range(H_kv):
            fill_normal(kc[b, hk, :n], 1000 + 16 * b + hk)
            fill_normal(vc[b, hk, :n], 2000 + 16 * b + hk)
    q = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    fill_normal(q, 150)
    o, lse = lib.decode(q, kc, vc, torch.tensor(kv_len, dtype=torch.int32, device="cuda"), scale)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        n = kv_len[b]
        ro, rl = orc.attention_decode(f64(q[b:b + 1]), f64(kc[b:b + 1, :, :n]), f64(vc[b:b + 1, :, :n]), [n], scale)
        assert max_err(o[b:b + 1], ro) <= TOL_BF16, b
        assert float(np.max(np.abs(lse[b:b + 1].cpu().numpy() - rl))) <= TOL_BF16, b
    del kc, vc, q, o, lse
    release()


def test_paged_decode_pages_past_4gib(lib):
    # [36000, 8, 64, 128] bf16 pages: 4.4 GiB each; the sequences use pages on both sides of 4 GiB.
    P, H, H_kv, ps, d = 36000, 32, 8, 64, 128
    assert P * H_kv * ps * d * 2 > 4 * GIB
    kv_len = [3000, 64, 4500]
    B = len(kv_len)
    max_pages = max((n + ps - 1) // ps for n in kv_len)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([160, 0])))
    page_ids = g.permutation(np.arange(P - 4000, P))[:B * max_pages]  # pages past 4 GiB
    page_ids[:8] = np.arange(8) * 17  # ... and a few near the start
    table = page_ids.reshape(B, max_pages).astype(np.int32)
    scale = 1.0 / math.sqrt(d)
    print("large paged decode: allocating", flush=True)
    kp = torch.empty((P, H_kv, ps, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    for b, n in enumerate(kv_len):  # only the pages below kv_len hold data
        for j in range((n + ps - 1) // ps):
            p = int(table[b, j])
            fill_normal(kp[p], 3000 + p)
            fill_normal(vp[p], 4000 + p)
    q = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    fill_normal(q, 170)
    o, lse = lib.decode_paged(q, kp, vp, torch.from_numpy(table).cuda(),
                              torch.tensor(kv_len, dtype=torch.int32, device="cuda"), scale)
    torch.cuda.synchronize()
    for b, n in enumerate(kv_len):
        used = table[b, :(n + ps - 1) // ps]
        kh = torch.cat([kp[int(p)] for p in used], dim=1)[:, :n].unsqueeze(0)  # [1, H_kv, n, d]
        vh = torch.cat([vp[int(p)] for p in used], dim=1)[:, :n].unsqueeze(0)
        ro, rl = orc.attention_decode(f64(q[b:b + 1]), f64(kh), f64(vh), [n], scale)
        assert max_err(o[b:b + 1], ro) <= TOL_BF16, b
        assert float(np.max(np.abs(lse[b:b + 1].cpu().numpy() - rl))) <= TOL_BF16, b
    del kp, vp, q, o, lse
    release()
