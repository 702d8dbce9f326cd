"""Parity of the HIP path (through the C ABI) with the fp64 oracle on the same seeded inputs.

Tolerances (max abs error per output tensor): 1e-5 on the float32 path, 2e-2 on the bf16 path
with fp32 accumulation. Small cases are compared element by element at sizes that span several
tiles and a ragged tail; the full-size workloads are compared on every element the oracle can
afford (all of the 1k causal prefill and the decode batch) or on sampled rows and heads.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as orc
from roofline_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def dev(t):
    return t.to("cuda")


def f64(t):
    return I.to_f64(t)


def max_err(gpu, ref):
    return float(np.max(np.abs(f64(gpu) - ref))) if ref.size else 0.0


def run_fwd(lib, w, causal=None):
    t = I.make_prefill(w, with_dout=False)
    causal = w.causal if causal is None else causal
    o, lse = lib.fwd(dev(t["q"]), dev(t["k"]), dev(t["v"]), causal, w.scale)
    torch.cuda.synchronize()
    return t, o.cpu(), lse.cpu()


# ---------------------------------------------------------------------------- forward ----

def test_tiny_f32_workload(lib):
    w = I.WORKLOADS["tiny_f32"]
    t, o, lse = run_fwd(lib, w)
    ro, rl = orc.attention_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), w.causal, w.scale)
    assert max_err(o, ro) <= TOL_F32
    assert max_err(lse, rl) <= TOL_F32


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,H_kv,N,d", [(1, 2, 2, 333, 64), (2, 4, 2, 77, 128), (1, 3, 1, 1, 64),
                                           (1, 2, 2, 200, 128)])
def test_f32_shapes(lib, B, H, H_kv, N, d, causal):
    w = I.Workload("f32_case", "fwd", B, H, H_kv, N, d, "f32", causal, seed=11)
    t, o, lse = run_fwd(lib, w)
    ro, rl = orc.attention_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), causal, w.scale)
    assert max_err(o, ro) <= TOL_F32
    assert max_err(lse, rl) <= TOL_F32


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,H_kv,N,d", [(1, 2, 2, 333, 128), (1, 2, 2, 333, 64), (2, 8, 2, 200, 128),
                                           (1, 4, 1, 65, 64), (1, 2, 2, 1, 128), (1, 1, 1, 129, 128),
                                           (1, 2, 2, 512, 64), (1, 2, 2, 600, 128), (1, 1, 1, 257, 64)])
def test_bf16_shapes(lib, B, H, H_kv, N, d, causal):
    w = I.Workload("bf16_case", "fwd", B, H, H_kv, N, d, "bf16", causal, seed=12)
    t, o, lse = run_fwd(lib, w)
    ro, rl = orc.attention_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), causal, w.scale)
    assert max_err(o, ro) <= TOL_BF16
    assert max_err(lse, rl) <= TOL_BF16


def test_prefill_causal_1k_full(lib):
    w = I.WORKLOADS["prefill_causal_1k"]
    t, o, lse = run_fwd(lib, w)
    ro, rl = orc.attention_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), w.causal, w.scale)
    eo, el = max_err(o, ro), max_err(lse, rl)
    print(f"prefill_causal_1k: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_BF16


def sample_rows(B, H, N, n_rand, seed):
    rng = np.random.default_rng(seed)
    fixed = [(0, 0, 0), (0, 0, 1), (B - 1, H - 1, N - 1), (0, H - 1, 127), (0, H - 1, 128), (B - 1, 0, 63),
             (B - 1, 0, 64), (0, 1, N // 2), (B - 1, H // 2, N - 129)]
    rnd = np.stack([rng.integers(0, B, n_rand), rng.integers(0, H, n_rand), rng.integers(0, N, n_rand)], 1)
    return np.concatenate([np.array(fixed), rnd])


@pytest.mark.parametrize("name", ["prefill_4k_causal", "prefill_4k"])
def test_prefill_4k_sampled_rows_and_heads(lib, name):
    w = I.WORKLOADS[name]
    t, o, lse = run_fwd(lib, w)
    q, k, v = f64(t["q"]), f64(t["k"]), f64(t["v"])
    rows = sample_rows(w.B, w.H, w.N, 300, seed=3)
    ro, rl = orc.attention_fwd_rows(q, k, v, w.causal, w.scale, rows)
    og = f64(o)[rows[:, 0], rows[:, 1], rows[:, 2]]
    lg = f64(lse)[rows[:, 0], rows[:, 1], rows[:, 2]]
    # one whole head as well
    rh, rhl = orc.attention_fwd(q[1:2, 31:32], k[1:2, 31:32], v[1:2, 31:32], w.causal, w.scale)
    e = max(float(np.max(np.abs(og - ro))), float(np.max(np.abs(f64(o)[1:2, 31:32] - rh))))
    el = max(float(np.max(np.abs(lg - rl))), float(np.max(np.abs(f64(lse)[1:2, 31:32] - rhl))))
    print(f"{name}: max|dO|={e:.3e} max|dLSE|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_BF16
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_16k_sampled_rows(lib, causal):
    """A long sequence (128 query tiles, 64 causal pairs per head): sampled rows against the oracle."""
    w = I.Workload("prefill_16k", "fwd", 1, 2, 2, 16384, 128, "bf16", causal, seed=16, qk_factor=0.5)
    t, o, lse = run_fwd(lib, w)
    rows = sample_rows(w.B, w.H, w.N, 120, seed=16)
    ro, rl = orc.attention_fwd_rows(f64(t["q"]), f64(t["k"]), f64(t["v"]), causal, w.scale, rows)
    og = f64(o)[rows[:, 0], rows[:, 1], rows[:, 2]]
    lg = f64(lse)[rows[:, 0], rows[:, 1], rows[:, 2]]
    e, el = float(np.max(np.abs(og - ro))), float(np.max(np.abs(lg - rl)))
    print(f"prefill_16k causal={causal}: max|dO|={e:.3e} max|dLSE|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_BF16


def test_causal_row0_and_constant_v(lib):
    w = I.Workload("inv", "fwd", 1, 2, 2, 300, 128, "bf16", True, seed=13)
    t = I.make_prefill(w, with_dout=False)
    o, lse = lib.fwd(dev(t["q"]), dev(t["k"]), dev(t["v"]), True, w.scale)
    o = o.cpu()
    # row 0 attends to key 0 only: P = 1 exactly, so O[0] = V[0] (bf16 round trip of V is exact)
    assert torch.equal(o[:, :, 0], t["v"][:, :, 0])
    cv = t["v"][:, :, :1].expand_as(t["v"]).contiguous()
    o2, _ = lib.fwd(dev(t["q"]), dev(t["k"]), dev(cv), True, w.scale)
    assert float((o2.cpu().float() - cv.float()).abs().max()) <= TOL_BF16


def test_one_hot_selection(lib):
    N, d = 256, 128
    sel = torch.arange(N) % d
    k = torch.zeros(1, 1, N, d)
    k[0, 0, torch.arange(d), torch.arange(d)] = 1.0
    q = torch.zeros(1, 1, N, d)
    q[0, 0, torch.arange(N), sel] = 64.0
    v = torch.from_numpy(I.normal_block(14, 2, 0, 0, (N, d))).view(1, 1, N, d)
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    o, _ = lib.fwd(dev(q), dev(k), dev(v), False, 1.0)  # scale*c = 64 -> weight of others ~ N e^-64
    assert float((o.cpu().float()[0, 0] - v.float()[0, 0, sel]).abs().max()) <= TOL_BF16


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_score_jump_beyond_exp_range(lib, d, causal):
    # Every row's maximum sits in a late key tile and exceeds all earlier scores by 200 (scale 1):
    # 2^(200 log2 e) overflows fp32, so the reference maximum must be raised from the raw scores
    # of that tile, not from exponentials taken against the earlier one. Row i selects key
    # N/2 + i mod (N/2) (non-causal) or key i itself (causal, rows >= N/2).
    N = 256
    half = N // 2
    k = torch.zeros(1, 1, N, d)
    k[0, 0, half + torch.arange(half), torch.arange(half) % d] = 1.0
    q = torch.zeros(1, 1, N, d)
    q[0, 0, torch.arange(N), torch.arange(N) % d] = 200.0
    v = torch.from_numpy(I.normal_block(15, 2, 0, 0, (N, d))).view(1, 1, N, d)
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    o, lse = lib.fwd(dev(q), dev(k), dev(v), causal, 1.0)
    ro, rl = orc.attention_fwd(f64(q), f64(k), f64(v), causal, 1.0)
    assert np.isfinite(o.cpu().float().numpy()).all()
    assert max_err(o, ro) <= TOL_BF16
    assert float(np.max(np.abs(lse.cpu().numpy() - rl))) <= TOL_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_scores_rising_below_and_above_the_lazy_threshold(lib, causal):
    # Scores (log2 units) are 0 on keys 0..63, 7 on keys 64..255 (every probability near 2^7 against
    # the first reference, which stays: no raise) and 14 on keys 256..511 (a raise).
    N, d = 512, 128
    beta = torch.zeros(N)
    beta[64:256] = 7.0 * math.log(2.0)
    beta[256:] = 14.0 * math.log(2.0)
    k = torch.zeros(1, 1, N, d)
    k[0, 0, :, 0] = beta
    q = torch.zeros(1, 1, N, d)
    q[0, 0, :, 0] = 1.0
    v = torch.from_numpy(I.normal_block(16, 2, 0, 0, (N, d))).view(1, 1, N, d)
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    o, lse = lib.fwd(dev(q), dev(k), dev(v), causal, 1.0)
    ro, rl = orc.attention_fwd(f64(q), f64(k), f64(v), causal, 1.0)
    assert max_err(o, ro) <= TOL_BF16
    assert float(np.max(np.abs(lse.cpu().numpy() - rl))) <= TOL_BF16


def test_forward_is_deterministic(lib):
    w = I.Workload("det", "fwd", 2, 4, 4, 520, 128, "bf16", True, seed=15)
    t = I.make_prefill(w, with_dout=False)
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    o1, l1 = lib.fwd(q, k, v, True, w.scale)
    o2, l2 = lib.fwd(q, k, v, True, w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# --------------------------------------------------------------------- ragged prefill ----

def varlen_case(lib, w, lengths=None):
    t = I.make_varlen(w, lengths)
    o, lse = lib.fwd_varlen(dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["cu_seqlens"]), int(max(t["lengths"].max(), 1)),
                            w.causal, w.scale)
    torch.cuda.synchronize()
    return t, o.cpu(), lse.cpu()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv,d", [(4, 2, 128), (4, 4, 64), (8, 1, 128)])
def test_fwd_varlen_ragged_lengths(lib, H, H_kv, d, causal):
    w = I.Workload("vl", "varlen", 5, H, H_kv, 600, d, "bf16", causal, seed=21)
    t, o, lse = varlen_case(lib, w, lengths=[1, 255, 256, 257, 600])
    ro, rl = orc.attention_fwd_varlen(f64(t["q"]), f64(t["k"]), f64(t["v"]), t["cu_seqlens"].numpy(), causal,
                                      w.scale)
    assert max_err(o, ro) <= TOL_BF16
    assert max_err(lse, rl) <= TOL_BF16


def test_fwd_varlen_empty_sequences(lib):
    w = I.Workload("vl0", "varlen", 4, 2, 2, 700, 128, "bf16", True, seed=22)
    t, o, lse = varlen_case(lib, w, lengths=[0, 700, 0, 3])
    ro, rl = orc.attention_fwd_varlen(f64(t["q"]), f64(t["k"]), f64(t["v"]), t["cu_seqlens"].numpy(), True, w.scale)
    assert max_err(o, ro) <= TOL_BF16 and max_err(lse, rl) <= TOL_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_varlen_equal_lengths_match_dense_bitwise(lib, causal):
    # Same sequences through both layouts: the kernel does the same arithmetic, only the row
    # strides differ, so the outputs must be identical.
    B, H, H_kv, N, d = 3, 4, 2, 333, 128
    w = I.Workload("vld", "varlen", B, H, H_kv, N, d, "bf16", causal, seed=23)
    t, o, lse = varlen_case(lib, w, lengths=[N] * B)
    q = t["q"].view(B, N, H, d).permute(0, 2, 1, 3).contiguous()
    k = t["k"].view(B, N, H_kv, d).permute(0, 2, 1, 3).contiguous()
    v = t["v"].view(B, N, H_kv, d).permute(0, 2, 1, 3).contiguous()
    od, ld = lib.fwd(dev(q), dev(k), dev(v), causal, w.scale)
    assert torch.equal(o.view(B, N, H, d).permute(0, 2, 1, 3), od.cpu())
    assert torch.equal(lse.view(H, B, N).permute(1, 0, 2), ld.cpu())


def test_fwd_varlen_full_workload_sampled_rows(lib):
    w = I.WORKLOADS["prefill_varlen"]
    t, o, lse = varlen_case(lib, w)
    cu = t["cu_seqlens"].numpy()
    rng = np.random.default_rng(7)
    rows = []
    for b in range(w.B):  # first, last and two random rows of every sequence, random heads
        for i in (0, int(t["lengths"][b]) - 1, *rng.integers(0, t["lengths"][b], 2)):
            rows.append((int(cu[b]) + int(i), int(rng.integers(0, w.H))))
    rows = np.array(rows)
    ro, rl = orc.attention_fwd_varlen_rows(f64(t["q"]), f64(t["k"]), f64(t["v"]), cu, w.causal, w.scale, rows)
    eo = float(np.max(np.abs(f64(o[rows[:, 0], rows[:, 1]]) - ro)))
    el = float(np.max(np.abs(f64(lse[rows[:, 1], rows[:, 0]]) - rl)))
    print(f"prefill_varlen: {len(rows)} rows, max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_BF16
    assert torch.isfinite(o.float()).all()


# ----------------------------------------------------------------------------- decode ----

def decode_check(lib, w, kv_len=None, n_seq_check=None):
    t = I.make_decode(w)
    if kv_len is not None:
        t = I.make_decode(w, nan_pad=False)
        t["kv_len"] = torch.tensor(kv_len, dtype=torch.int32)
        for b in range(w.B):
            t["k"][b, :, kv_len[b]:] = float("nan")
            t["v"][b, :, kv_len[b]:] = float("nan")
    o, lse = lib.decode(dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["kv_len"]), w.scale)
    o, lse = o.cpu(), lse.cpu()
    q = f64(t["q"])
    lens = t["kv_len"].numpy()
    err_o = err_l = 0.0
    seqs = range(w.B) if n_seq_check is None else range(min(w.B, n_seq_check))
    for b in seqs:
        n = int(lens[b])
        kb = f64(t["k"][b:b + 1, :, :n])
        vb = f64(t["v"][b:b + 1, :, :n])
        ro, rl = orc.attention_decode(q[b:b + 1], kb, vb, np.array([n]), w.scale)
        err_o = max(err_o, float(np.max(np.abs(f64(o[b:b + 1]) - ro))))
        err_l = max(err_l, float(np.max(np.abs(f64(lse[b:b + 1]) - rl))))
    return err_o, err_l


def test_decode_gqa_full_workload(lib):
    w = I.WORKLOADS["decode_gqa"]
    eo, el = decode_check(lib, w)
    print(f"decode_gqa: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_BF16


# Group sizes 1, 2, 4, 8 have kernels of their own; 3, 7, 16 run the 16-column kernel in one
# chunk, 40 in three (16 + 16 + 8 query heads).
@pytest.mark.parametrize("H,H_kv,d", [(8, 8, 128), (8, 4, 64), (16, 4, 128), (16, 2, 128), (8, 1, 64),
                                      (12, 4, 128), (14, 2, 64), (16, 1, 128), (40, 1, 128)])
def test_decode_ragged_lengths(lib, H, H_kv, d):
    w = I.Workload("dec", "decode", 7, H, H_kv, 1100, d, "bf16", False, seed=16, kv_lo=1, kv_hi=1100)
    eo, el = decode_check(lib, w, kv_len=[1, 255, 257, 1023, 1024, 1025, 1100])
    assert eo <= TOL_BF16 and el <= TOL_BF16


def test_decode_more_than_64_splits(lib):
    # About 69 and 65 partial records per (sequence, head) (every workgroup share holds at least
    # 1024 keys): the merge takes more than one 64-lane pass over the records.
    w = I.Workload("dec_long", "decode", 2, 8, 2, 70000, 64, "bf16", False, seed=18, kv_lo=1, kv_hi=70000)
    eo, el = decode_check(lib, w, kv_len=[70000, 65601])
    assert eo <= TOL_BF16 and el <= TOL_BF16


def decode_check_with_empty(lib, w, lens):
    """Decode with the given lengths (zeros allowed): empty sequences give O = 0 and LSE = -inf
    exactly, the others match the oracle."""
    t = I.make_decode(w, nan_pad=False)
    t["kv_len"] = torch.tensor(lens, dtype=torch.int32)
    for b in range(w.B):
        t["k"][b, :, lens[b]:] = float("nan")
        t["v"][b, :, lens[b]:] = float("nan")
    o, lse = lib.decode(dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["kv_len"]), w.scale)
    o, lse = o.cpu(), lse.cpu()
    q = f64(t["q"])
    err = 0.0
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(o[b]) == 0 and bool(torch.all(lse[b] == -float("inf")))
            continue
        ro, rl = orc.attention_decode(q[b:b + 1], f64(t["k"][b:b + 1, :, :n]), f64(t["v"][b:b + 1, :, :n]),
                                      np.array([n]), w.scale)
        err = max(err, float(np.max(np.abs(f64(o[b:b + 1]) - ro))), float(np.max(np.abs(f64(lse[b:b + 1]) - rl))))
    return err


def test_decode_one_share_over_many_short_sequences(lib):
    # 40 sequences of 0..40 keys over 2 KV heads: fewer than 1024 keys in all, so one workgroup
    # takes every segment, one piece (and one merge) after another, empty sequences skipped.
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(0, 41, size=40)]
    lens[3] = lens[17] = 0
    w = I.Workload("dec_short", "decode", 40, 8, 2, 64, 128, "bf16", False, seed=41, kv_lo=0, kv_hi=40)
    assert decode_check_with_empty(lib, w, lens) <= TOL_BF16


def test_decode_more_than_64_sequences(lib):
    # 130 sequences (three 64-lane chunks of the length scan) with mixed lengths, zeros included:
    # workgroup shares start and end inside sequences of every chunk.
    rng = np.random.default_rng(42)
    lens = [int(x) for x in rng.integers(0, 2500, size=130)]
    lens[0] = lens[64] = lens[129] = 0
    lens[63], lens[65] = 2500, 1
    w = I.Workload("dec_many", "decode", 130, 8, 4, 2500, 64, "bf16", False, seed=42, kv_lo=0, kv_hi=2500)
    assert decode_check_with_empty(lib, w, lens) <= TOL_BF16


@pytest.mark.parametrize("page_size", [32, 64, 256])
@pytest.mark.parametrize("H,H_kv,d", [(8, 8, 128), (8, 4, 64), (16, 2, 128), (10, 2, 128), (32, 1, 64)])
def test_decode_paged_matches_dense_and_oracle(lib, H, H_kv, d, page_size):
    # Same rows as the contiguous cache, scattered over shuffled pages: the result must equal the
    # contiguous decode bit for bit (same arithmetic, other addresses) and the paged oracle.
    w = I.Workload("decp", "decode", 7, H, H_kv, 1100, d, "bf16", False, seed=16, kv_lo=1, kv_hi=1100)
    dense = I.make_decode(w, nan_pad=False)
    dense["kv_len"] = torch.tensor([1, 255, 257, 1023, 1024, 1025, 1100], dtype=torch.int32)
    for b in range(w.B):
        n = int(dense["kv_len"][b])
        dense["k"][b, :, n:] = float("nan")
        dense["v"][b, :, n:] = float("nan")
    t = I.make_decode_paged(w, page_size, dense=dense)
    o, lse = lib.decode_paged(dev(t["q"]), dev(t["k_pages"]), dev(t["v_pages"]), dev(t["block_table"]),
                              dev(t["kv_len"]), w.scale)
    od, lsed = lib.decode(dev(dense["q"]), dev(dense["k"]), dev(dense["v"]), dev(dense["kv_len"]), w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    assert torch.equal(o.cpu(), od.cpu()) and torch.equal(lse.cpu(), lsed.cpu())
    ro, rl = orc.attention_decode_paged(f64(t["q"]), t["k_pages"].float().numpy(), t["v_pages"].float().numpy(),
                                        t["block_table"].numpy(), t["kv_len"].numpy(), w.scale)
    assert max_err(o.cpu(), ro) <= TOL_BF16 and max_err(lse.cpu(), rl) <= TOL_BF16


def test_decode_paged_full_workload_matches_dense(lib):
    w = I.WORKLOADS["decode_gqa"]
    dense = I.make_decode(w)
    t = I.make_decode_paged(w, 64, dense=dense)
    o, lse = lib.decode_paged(dev(t["q"]), dev(t["k_pages"]), dev(t["v_pages"]), dev(t["block_table"]),
                              dev(t["kv_len"]), w.scale)
    od, lsed = lib.decode(dev(dense["q"]), dev(dense["k"]), dev(dense["v"]), dev(dense["kv_len"]), w.scale)
    assert torch.equal(o.cpu(), od.cpu()) and torch.equal(lse.cpu(), lsed.cpu())
    assert torch.isfinite(o.float()).all()


def test_decode_workspace_reuse_with_other_inputs(lib):
    # One workspace serves calls on different inputs (contiguous and paged, one sequence of length
    # 0, lengths on both sides of 1024 keys): each call's records, piece counts included, are
    # written before the merge reads them, so no call sees another's partial results.
    lens = [5000, 1, 1024, 1025, 3333, 0]
    cases = []
    for seed in (19, 20):
        w = I.Workload("decws", "decode", 6, 16, 4, 5000, 128, "bf16", False, seed=seed, kv_lo=1, kv_hi=5000)
        t = I.make_decode(w, nan_pad=False)
        t["kv_len"] = torch.tensor(lens, dtype=torch.int32)
        cases.append((w, t, {k: dev(x) for k, x in t.items()}))
    w = cases[0][0]
    ws = torch.full((lib.decode_workspace_size(w.B, w.H, w.N, w.d),), 0x7F, dtype=torch.uint8, device="cuda")
    outs = {0: [], 1: []}
    for rep in range(3):
        for i, (w, t, g) in enumerate(cases):
            o, lse = lib.decode(g["q"], g["k"], g["v"], g["kv_len"], w.scale, workspace=ws)
            outs[i].append((o.cpu(), lse.cpu()))
    for i, (w, t, g) in enumerate(cases):
        o0, l0 = outs[i][0]
        for o, lse in outs[i][1:]:
            assert torch.equal(o, o0) and torch.equal(lse, l0)
        tp = I.make_decode_paged(w, 128, dense=t)
        op, lsep = lib.decode_paged(dev(tp["q"]), dev(tp["k_pages"]), dev(tp["v_pages"]), dev(tp["block_table"]),
                                    dev(tp["kv_len"]), w.scale, workspace=ws)
        assert torch.equal(op.cpu(), o0) and torch.equal(lsep.cpu(), l0)
        q = f64(t["q"])
        for b, n in enumerate(lens):
            if n == 0:
                assert torch.all(o0[b] == 0) and torch.all(torch.isneginf(l0[b]))
                continue
            ro, rl = orc.attention_decode(q[b:b + 1], f64(t["k"][b:b + 1, :, :n]), f64(t["v"][b:b + 1, :, :n]),
                                          np.array([n]), w.scale)
            assert max_err(o0[b:b + 1], ro) <= TOL_BF16 and max_err(l0[b:b + 1], rl) <= TOL_BF16


def test_decode_zero_length_is_defined(lib):
    w = I.Workload("dec0", "decode", 2, 4, 4, 64, 128, "bf16", False, seed=17, kv_lo=1, kv_hi=64)
    t = I.make_decode(w)
    kv = torch.tensor([0, 5], dtype=torch.int32)
    o, lse = lib.decode(dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(kv), w.scale)
    o, lse = o.cpu(), lse.cpu()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.isfinite(o[1].float()).all()


# --------------------------------------------------------------------------- backward ----

def bwd_case(lib, w):
    t = I.make_prefill(w, with_dout=True)
    q, k, v, do = dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["do"])
    o, lse = lib.fwd(q, k, v, w.causal, w.scale)
    dq, dk, dv = lib.bwd(q, k, v, o, do, lse, w.causal, w.scale)
    torch.cuda.synchronize()
    return t, o.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,H_kv,N,d", [(1, 2, 2, 256, 128), (1, 2, 2, 200, 128), (2, 2, 2, 333, 64),
                                           (1, 1, 1, 1, 128), (1, 2, 2, 65, 64),
                                           # grouped heads: dK/dV sum over each KV head's query heads
                                           (1, 4, 2, 600, 128), (2, 8, 2, 333, 64), (1, 4, 1, 200, 128),
                                           (1, 8, 1, 129, 64)])
def test_bwd_shapes(lib, B, H, H_kv, N, d, causal):
    w = I.Workload("bwd_case", "fwdbwd", B, H, H_kv, N, d, "bf16", causal, seed=18)
    t, o, dq, dk, dv = bwd_case(lib, w)
    rdq, rdk, rdv, ro, _ = orc.attention_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]), causal, w.scale)
    errs = [max_err(o, ro), max_err(dq, rdq), max_err(dk, rdk), max_err(dv, rdv)]
    assert max(errs) <= TOL_BF16, errs


def test_fwdbwd_4k_causal_sampled_heads(lib):
    w = I.WORKLOADS["fwdbwd_4k_causal"]
    t, o, dq, dk, dv = bwd_case(lib, w)
    worst = [0.0] * 4
    for b, h in ((0, 0), (1, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rdq, rdk, rdv, ro, _ = orc.attention_bwd(f64(t["q"][sl]), f64(t["k"][sl]), f64(t["v"][sl]),
                                                 f64(t["do"][sl]), w.causal, w.scale)
        errs = [max_err(o[sl], ro), max_err(dq[sl], rdq), max_err(dk[sl], rdk), max_err(dv[sl], rdv)]
        worst = [max(a, e) for a, e in zip(worst, errs)]
    print(f"fwdbwd_4k_causal: max|dO|,|ddQ|,|ddK|,|ddV| = {worst}")
    assert max(worst) <= TOL_BF16, worst
    for x in (dq, dk, dv):
        assert torch.isfinite(x).all()


# ------------------------------------------------------------------- ragged backward ----

def varlen_bwd_case(lib, w, lengths=None):
    t = I.make_varlen(w, lengths, with_dout=True)
    q, k, v, do, cu = dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["do"]), dev(t["cu_seqlens"])
    max_len = int(max(t["lengths"].max(), 1))
    o, lse = lib.fwd_varlen(q, k, v, cu, max_len, w.causal, w.scale)
    dq, dk, dv = lib.bwd_varlen(q, k, v, o, do, lse, cu, max_len, w.causal, w.scale)
    torch.cuda.synchronize()
    return t, o.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv,d", [(4, 2, 128), (4, 4, 64), (8, 1, 128)])
def test_bwd_varlen_ragged_lengths(lib, H, H_kv, d, causal):
    # lengths straddling the 64/128-row tiles: 1, one short of, at and past a tile edge, and more
    w = I.Workload("vlb", "varlen", 5, H, H_kv, 600, d, "bf16", causal, seed=24)
    t, o, dq, dk, dv = varlen_bwd_case(lib, w, lengths=[1, 255, 256, 257, 600])
    rdq, rdk, rdv, ro, _ = orc.attention_bwd_varlen(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]),
                                                    t["cu_seqlens"].numpy(), causal, w.scale)
    errs = [max_err(o, ro), max_err(dq, rdq), max_err(dk, rdk), max_err(dv, rdv)]
    assert max(errs) <= TOL_BF16, errs


def test_bwd_varlen_empty_sequences(lib):
    w = I.Workload("vlb0", "varlen", 4, 4, 2, 700, 128, "bf16", True, seed=25)
    t, o, dq, dk, dv = varlen_bwd_case(lib, w, lengths=[0, 700, 0, 3])
    rdq, rdk, rdv, _, _ = orc.attention_bwd_varlen(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]),
                                                   t["cu_seqlens"].numpy(), True, w.scale)
    errs = [max_err(dq, rdq), max_err(dk, rdk), max_err(dv, rdv)]
    assert max(errs) <= TOL_BF16, errs


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_equal_lengths_match_dense_bitwise(lib, causal):
    # Equal lengths through both layouts: every gradient element comes from the same arithmetic in
    # the same order (only the row strides and the work-item order differ), so the results match
    # bit for bit.
    B, H, H_kv, N, d = 3, 4, 2, 333, 128
    w = I.Workload("vlbd", "varlen", B, H, H_kv, N, d, "bf16", causal, seed=26)
    t, o, dq, dk, dv = varlen_bwd_case(lib, w, lengths=[N] * B)
    dense = lambda x, h: dev(x.view(B, N, h, d).permute(0, 2, 1, 3).contiguous())
    q, k, v, do = dense(t["q"], H), dense(t["k"], H_kv), dense(t["v"], H_kv), dense(t["do"], H)
    od, ld = lib.fwd(q, k, v, causal, w.scale)
    gd = lib.bwd(q, k, v, od, do, ld, causal, w.scale)
    packed = lambda x, h: x.view(B, N, h, d).permute(0, 2, 1, 3)
    assert torch.equal(packed(o, H), od.cpu())
    for got, ref, h in zip((dq, dk, dv), gd, (H, H_kv, H_kv)):
        assert torch.equal(packed(got, h), ref.cpu())


def test_bwd_varlen_full_workload_sampled_sequences(lib):
    # The ragged prefill workload (16 sequences of 512-8192 tokens, H 32 / H_kv 8, causal): the
    # gradients of whole sequences and KV groups, which the oracle computes on those rows alone.
    w = I.WORKLOADS["prefill_varlen"]
    t, o, dq, dk, dv = varlen_bwd_case(lib, w)
    cu, lengths = t["cu_seqlens"].numpy(), t["lengths"]
    g = w.H // w.H_kv
    order = np.argsort(lengths)
    picks = [(int(order[0]), hk) for hk in range(w.H_kv)]  # the shortest sequence, every KV group
    mid = int(order[min(np.searchsorted(lengths[order], 4096), len(order) - 1)])  # near 4096 tokens
    picks += [(mid, 0), (mid, w.H_kv - 1)]
    worst = [0.0] * 3
    for b, hk in picks:
        r = slice(int(cu[b]), int(cu[b + 1]))
        hq = slice(hk * g, (hk + 1) * g)
        sub = lambda x, hs: f64(x[r, hs])
        rdq, rdk, rdv, _, _ = orc.attention_bwd_varlen(sub(t["q"], hq), sub(t["k"], slice(hk, hk + 1)),
                                                       sub(t["v"], slice(hk, hk + 1)), sub(t["do"], hq),
                                                       [0, r.stop - r.start], True, w.scale)
        errs = [max_err(dq[r, hq], rdq), max_err(dk[r, hk:hk + 1], rdk), max_err(dv[r, hk:hk + 1], rdv)]
        worst = [max(a, e) for a, e in zip(worst, errs)]
    print(f"prefill_varlen bwd: sequences {sorted({b for b, _ in picks})}, max|ddQ|,|ddK|,|ddV| = {worst}")
    assert max(worst) <= TOL_BF16, worst
    for x in (dq, dk, dv):
        assert torch.isfinite(x).all()


def test_varlen_malformed_offsets_stay_in_bounds(lib):
    # Offsets that decrease, pass T or go negative are clamped on the device, so the kernels read
    # and write only inside the tensors. Sequence 0 owns rows 0..149 alone (sequence 2, clamped to
    # rows 150..699, overlaps its tail; sequences 1 and 3 clamp to empty): O, LSE and dQ of those
    # rows depend on no other row's results and stay exact. (dK, dV of its keys also use query rows
    # 150..199, whose O and LSE both sequences write.)
    H, H_kv, d, T = 4, 2, 128, 700
    w = I.Workload("vlbad", "varlen", 2, H, H_kv, 600, d, "bf16", True, seed=27)
    t = I.make_varlen(w, lengths=[200, 500], with_dout=True)
    q, k, v, do = dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["do"])
    cu = torch.tensor([0, 200, 150, 900, -5], dtype=torch.int32, device="cuda")
    o, lse = lib.fwd_varlen(q, k, v, cu, 600, True, w.scale)
    dq, dk, dv = lib.bwd_varlen(q, k, v, o, do, lse, cu, 600, True, w.scale)
    torch.cuda.synchronize()
    r = slice(0, 150)
    rdq, _, _, ro, rl = orc.attention_bwd_varlen(f64(t["q"][:200]), f64(t["k"][:200]), f64(t["v"][:200]),
                                                 f64(t["do"][:200]), [0, 200], True, w.scale)
    errs = [max_err(o[r].cpu(), ro[r]), max_err(lse[:, r].cpu(), rl[:, r]), max_err(dq[r].cpu(), rdq[r])]
    assert max(errs) <= TOL_BF16, errs
    for x in (o, dq, dk, dv):  # every row belongs to some clamped sequence and holds finite values
        assert bool(torch.isfinite(x.float()).all())


def test_varlen_max_seqlen_truncates_longer_sequences(lib):
    # A sequence longer than max_seqlen is treated as its first max_seqlen rows; its other rows are
    # not written. Sequence 0 (300 rows) runs as a 256-row sequence, sequence 1 (400 rows) as rows
    # 300..555.
    H, H_kv, d = 2, 1, 64
    w = I.Workload("vltr", "varlen", 2, H, H_kv, 400, d, "bf16", False, seed=28)
    t = I.make_varlen(w, lengths=[300, 400], with_dout=True)
    q, k, v, do = dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["do"])
    cu = dev(t["cu_seqlens"])
    sentinel = 4096.0  # exact in bf16 and fp32
    o = torch.full_like(q, sentinel)
    o, lse = lib.fwd_varlen(q, k, v, cu, 256, False, w.scale, out=o)
    dq = torch.full(q.shape, sentinel, dtype=torch.float32, device="cuda")
    dk = torch.full(k.shape, sentinel, dtype=torch.float32, device="cuda")
    dv = torch.full(v.shape, sentinel, dtype=torch.float32, device="cuda")
    lib.bwd_varlen(q, k, v, o, do, lse, cu, 256, False, w.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for a, e in ((0, 256), (300, 556)):
        r = slice(a, e)
        rdq, rdk, rdv, ro, _ = orc.attention_bwd_varlen(f64(t["q"][r]), f64(t["k"][r]), f64(t["v"][r]),
                                                        f64(t["do"][r]), [0, e - a], False, w.scale)
        errs = [max_err(o[r].cpu(), ro), max_err(dq[r].cpu(), rdq), max_err(dk[r].cpu(), rdk),
                max_err(dv[r].cpu(), rdv)]
        assert max(errs) <= TOL_BF16, (a, errs)
    for x in (o, dq, dk, dv):  # rows past each truncated sequence keep the sentinel
        assert bool((x[256:300].float() == sentinel).all()) and bool((x[556:].float() == sentinel).all())


def test_bwd_is_deterministic(lib):
    w = I.Workload("bdet", "fwdbwd", 1, 4, 4, 384, 128, "bf16", True, seed=19)
    t = I.make_prefill(w, with_dout=True)
    q, k, v, do = dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["do"])
    o, lse = lib.fwd(q, k, v, True, w.scale)
    a = lib.bwd(q, k, v, o, do, lse, True, w.scale)
    b = lib.bwd(q, k, v, o, do, lse, True, w.scale)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_timer_reports_kernels(lib):
    w = I.Workload("tm", "fwd", 1, 2, 2, 256, 128, "bf16", True, seed=20)
    t = I.make_prefill(w, with_dout=False)
    lib.timing_reset()
    lib.timing_enable(True)
    try:
        for _ in range(3):
            lib.fwd(dev(t["q"]), dev(t["k"]), dev(t["v"]), True, w.scale)
    finally:
        lib.timing_enable(False)
    rec = lib.timing_read()
    smp = lib.timing_samples()
    lib.timing_reset()
    assert rec["fwd_bf16_d128_causal"][0] == 3 and rec["fwd_bf16_d128_causal"][1] > 0
    # one duration per launch, summing to the total
    per = smp["fwd_bf16_d128_causal"]
    assert len(per) == 3 and all(x > 0 for x in per)
    assert abs(sum(per) - rec["fwd_bf16_d128_causal"][1]) <= 1e-3 * rec["fwd_bf16_d128_causal"][1]
    # releasing the events leaves the library usable: the timer creates new ones
    lib.release()
    lib.timing_enable(True)
    try:
        lib.fwd(dev(t["q"]), dev(t["k"]), dev(t["v"]), True, w.scale)
    finally:
        lib.timing_enable(False)
    assert lib.timing_read()["fwd_bf16_d128_causal"][0] == 1
    lib.release()
