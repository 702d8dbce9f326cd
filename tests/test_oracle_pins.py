"""Pins for the fp64 oracle, each tied to something other than the oracle itself.

Kinds of pin used (none re-types the oracle's formula):
  * library routine: torch's scaled_dot_product_attention and autograd in float64
    on the CPU, an implementation that shares no code with the oracle;
  * closed forms: scale = 0 (uniform weights), N = 1, a one-hot construction
    whose log-sum-exp has an exact value;
  * invariants the pages fix ("Why Fast GPUs Still Wait for Memory", section
    "Attention from first principles"): softmax rows sum to one, a constant V
    gives a constant output, causal row 0 equals V[0], a large-scaled one-hot
    Q.K selects one V row; plus permutation and shift invariance;
  * brute force: central finite differences of L = sum(O * dO) on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as orc

RNG = np.random.default_rng(12345)


def rand(*shape):
    return RNG.standard_normal(shape)


def sdpa(q, k, v, causal, scale):
    """torch float64 CPU reference, with KV heads expanded for grouped queries."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1)
    vt = vt.repeat_interleave(g, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale).numpy()


# ---------------------------------------------------------------- forward ---

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,H_kv,N,d", [(1, 2, 2, 128, 64), (2, 4, 2, 37, 16), (1, 8, 1, 65, 32), (2, 3, 3, 1, 8)])
def test_fwd_matches_torch_sdpa(B, H, H_kv, N, d, causal):
    q, k, v = rand(B, H, N, d), rand(B, H_kv, N, d), rand(B, H_kv, N, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = orc.attention_fwd(q, k, v, causal, scale)
    np.testing.assert_allclose(o, sdpa(q, k, v, causal, scale), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_scale_zero_is_uniform_average(causal):
    B, H, N, d = 1, 2, 50, 8
    q, k, v = rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d)
    o, lse = orc.attention_fwd(q, k, v, causal, 0.0)
    if causal:
        counts = np.arange(1, N + 1)
        want = np.cumsum(v, axis=2) / counts[None, None, :, None]
        want_lse = np.broadcast_to(np.log(counts), lse.shape)
    else:
        want = np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape)
        want_lse = np.full(lse.shape, math.log(N))
    np.testing.assert_allclose(o, want, atol=1e-13)
    np.testing.assert_allclose(lse, want_lse, atol=1e-13)


def test_fwd_single_key():
    q, k, v = rand(1, 3, 1, 16), rand(1, 3, 1, 16), rand(1, 3, 1, 16)
    scale = 0.37
    o, lse = orc.attention_fwd(q, k, v, False, scale)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse[..., 0], scale * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), atol=1e-14)


def test_fwd_rows_sum_to_one():
    # With V the identity (d = N), O = P itself.
    N = 48
    q, k = rand(1, 2, N, N), rand(1, 2, N, N)
    v = np.broadcast_to(np.eye(N), (1, 2, N, N)).copy()
    for causal in (False, True):
        p, _ = orc.attention_fwd(q, k, v, causal, 0.2)
        assert (p >= 0).all()
        np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-13)
        if causal:
            assert np.all(np.triu(p[0, 0], k=1) == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_constant_v(causal):
    N, d = 64, 16
    q, k = rand(1, 2, N, d), rand(1, 2, N, d)
    c = rand(d)
    v = np.broadcast_to(c, (1, 2, N, d)).copy()
    o, _ = orc.attention_fwd(q, k, v, causal, 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-13)


def test_fwd_causal_row0():
    q, k, v = rand(2, 2, 40, 16), rand(2, 2, 40, 16), rand(2, 2, 40, 16)
    scale = 0.3
    o, lse = orc.attention_fwd(q, k, v, True, scale)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], scale * np.sum(q[:, :, 0] * k[:, :, 0], -1), atol=1e-14)


def one_hot_case(N, d, c, scale, perm_seed=0):
    """k_j = e_j (j < d), 0 otherwise; q_i = c e_sigma(i); so S_ij = scale*c*[j == sigma(i)]."""
    k = np.zeros((1, 1, N, d))
    k[0, 0, np.arange(d), np.arange(d)] = 1.0
    sigma = np.random.default_rng(perm_seed).integers(0, d, size=N)
    q = np.zeros((1, 1, N, d))
    q[0, 0, np.arange(N), sigma] = c
    v = rand(1, 1, N, d)
    return q, k, v, sigma


def test_fwd_one_hot_selection_and_exact_lse():
    N, d, c, scale = 128, 64, 600.0, 0.125  # scale * c = 75
    q, k, v, sigma = one_hot_case(N, d, c, scale)
    o, lse = orc.attention_fwd(q, k, v, False, scale)
    np.testing.assert_allclose(o[0, 0], v[0, 0, sigma], atol=N * math.exp(-75) * 10)
    # lse_i = ln(e^{scale c} + (N - 1) e^0), a closed form
    np.testing.assert_allclose(lse[0, 0], scale * c + math.log1p((N - 1) * math.exp(-scale * c)), rtol=1e-15)
    # a small logit gap: exact weights e^{a}/(e^{a}+N-1) on the selected row, 1/(e^a+N-1) elsewhere
    a = 1.5
    o2, lse2 = orc.attention_fwd(q * (a / (scale * c)), k, v, False, scale)
    z = math.exp(a) + N - 1
    want = (v[0, 0].sum(axis=0)[None, :] + (math.exp(a) - 1.0) * v[0, 0, sigma]) / z
    np.testing.assert_allclose(o2[0, 0], want, atol=1e-13)
    np.testing.assert_allclose(lse2[0, 0], math.log(z), atol=1e-14)


def test_fwd_permutation_invariance():
    N, d = 33, 8
    q, k, v = rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d)
    o, lse = orc.attention_fwd(q, k, v, False, 0.4)
    pk = RNG.permutation(N)
    pq = RNG.permutation(N)
    o2, lse2 = orc.attention_fwd(q[:, :, pq], k[:, :, pk], v[:, :, pk], False, 0.4)
    np.testing.assert_allclose(o2, o[:, :, pq], atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, :, pq], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_key_shift_moves_lse_only(causal):
    # Adding u to every key adds scale*q_i.u to the whole score row i.
    N, d, scale = 40, 8, 0.3
    q, k, v = rand(1, 2, N, d), rand(1, 2, N, d), rand(1, 2, N, d)
    u = rand(d)
    o, lse = orc.attention_fwd(q, k, v, causal, scale)
    o2, lse2 = orc.attention_fwd(q, k + u, v, causal, scale)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + scale * (q @ u), atol=1e-12)


def test_fwd_gqa_equals_expanded_heads():
    B, H, H_kv, N, d = 1, 8, 2, 20, 8
    q, k, v = rand(B, H, N, d), rand(B, H_kv, N, d), rand(B, H_kv, N, d)
    o, lse = orc.attention_fwd(q, k, v, True, 0.3)
    # query heads 0..3 read KV head 0, heads 4..7 read KV head 1
    o_a, lse_a = orc.attention_fwd(q[:, :4], k[:, :1], v[:, :1], True, 0.3)
    np.testing.assert_array_equal(o[:, :4], o_a)
    o_b, _ = orc.attention_fwd(q[:, 4:], k[:, 1:], v[:, 1:], True, 0.3)
    np.testing.assert_array_equal(o[:, 4:], o_b)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_rows_agree_with_full(causal):
    B, H, H_kv, N, d = 2, 4, 2, 70, 16
    q, k, v = rand(B, H, N, d), rand(B, H_kv, N, d), rand(B, H_kv, N, d)
    o, lse = orc.attention_fwd(q, k, v, causal, 0.25)
    rows = np.array([[0, 0, 0], [1, 3, 69], [0, 2, 35], [1, 1, 1]])
    o_r, lse_r = orc.attention_fwd_rows(q, k, v, causal, 0.25, rows)
    np.testing.assert_allclose(o_r, o[rows[:, 0], rows[:, 1], rows[:, 2]], atol=1e-13)
    np.testing.assert_allclose(lse_r, lse[rows[:, 0], rows[:, 1], rows[:, 2]], atol=1e-13)
    np.testing.assert_allclose(o_r, sdpa(q, k, v, causal, 0.25)[rows[:, 0], rows[:, 1], rows[:, 2]], atol=1e-12)


# ----------------------------------------------------------------- decode ---

def test_decode_matches_sdpa_single_query_and_ignores_pad():
    B, H, H_kv, N_cap, d = 3, 8, 2, 50, 16
    q = rand(B, H, d)
    kc, vc = rand(B, H_kv, N_cap, d), rand(B, H_kv, N_cap, d)
    kv_len = np.array([1, 17, 50])
    for b in range(B):
        kc[b, :, kv_len[b]:] = np.nan
        vc[b, :, kv_len[b]:] = np.nan
    scale = 0.25
    o, lse = orc.attention_decode(q, kc, vc, kv_len, scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    for b in range(B):
        n = kv_len[b]
        want = sdpa(q[b][None, :, None, :], kc[b][None, :, :n], vc[b][None, :, :n], False, scale)
        np.testing.assert_allclose(o[b], want[0, :, 0], atol=1e-12)
    # length 1 gives that row's V exactly
    np.testing.assert_array_equal(o[0], np.repeat(vc[0, :, 0], H // H_kv, axis=0))


def test_decode_is_last_causal_row():
    B, H, H_kv, N, d = 1, 4, 1, 30, 8
    q, k, v = rand(B, H, N, d), rand(B, H_kv, N, d), rand(B, H_kv, N, d)
    o, lse = orc.attention_fwd(q, k, v, True, 0.3)
    od, lsed = orc.attention_decode(q[:, :, -1], k, v, np.array([N]), 0.3)
    np.testing.assert_allclose(od, o[:, :, -1], atol=1e-13)
    np.testing.assert_allclose(lsed, lse[:, :, -1], atol=1e-13)


def to_pages(kc, page_size, order):
    """Cut a contiguous cache [B,H_kv,N_cap,d] into pages [P,H_kv,ps,d] placed at `order`."""
    B, H_kv, N_cap, d = kc.shape
    per = N_cap // page_size
    pages = np.full((B * per, H_kv, page_size, d), np.nan)
    table = np.empty((B, per), dtype=np.int64)
    for b in range(B):
        for j in range(per):
            phys = order[b * per + j]
            pages[phys] = kc[b, :, j * page_size:(j + 1) * page_size]
            table[b, j] = phys
    return pages, table


@pytest.mark.parametrize("shuffle", [False, True])
def test_decode_paged_equals_contiguous(shuffle):
    # In-order pages of a contiguous cache, or the same pages scattered in physical memory, give
    # the dense decode's result; unused pages and the unused tail of a last page are NaN.
    B, H, H_kv, N_cap, d, ps = 3, 8, 2, 48, 8, 16
    q = rand(B, H, d)
    kc, vc = rand(B, H_kv, N_cap, d), rand(B, H_kv, N_cap, d)
    kv_len = np.array([1, 17, 48])
    for b in range(B):
        kc[b, :, kv_len[b]:] = np.nan
        vc[b, :, kv_len[b]:] = np.nan
    order = RNG.permutation(B * N_cap // ps) if shuffle else np.arange(B * N_cap // ps)
    kp, table = to_pages(kc, ps, order)
    vp, _ = to_pages(vc, ps, order)
    kp = np.concatenate([kp, np.full((2, H_kv, ps, d), np.nan)])  # pages no sequence references
    vp = np.concatenate([vp, np.full((2, H_kv, ps, d), np.nan)])
    o, lse = orc.attention_decode_paged(q, kp, vp, table, kv_len, 0.3)
    od, lsed = orc.attention_decode(q, kc, vc, kv_len, 0.3)
    np.testing.assert_array_equal(o, od)
    np.testing.assert_array_equal(lse, lsed)


def test_decode_paged_matches_sdpa():
    B, H, H_kv, d, ps = 2, 4, 1, 8, 4
    kp, vp = rand(7, H_kv, ps, d), rand(7, H_kv, ps, d)
    table = np.array([[5, 0, 3], [6, 2, 1]])
    kv_len = np.array([10, 12])
    q = rand(B, H, d)
    o, _ = orc.attention_decode_paged(q, kp, vp, table, kv_len, 0.5)
    for b in range(B):
        kb = torch.from_numpy(kp[table[b]].transpose(1, 0, 2, 3).reshape(H_kv, -1, d)[:, :kv_len[b]])
        vb = torch.from_numpy(vp[table[b]].transpose(1, 0, 2, 3).reshape(H_kv, -1, d)[:, :kv_len[b]])
        qb = torch.from_numpy(q[b])[:, None, :]
        want = torch.nn.functional.scaled_dot_product_attention(qb, kb.expand(H, -1, -1), vb.expand(H, -1, -1),
                                                                scale=0.5)[:, 0].numpy()
        np.testing.assert_allclose(o[b], want, atol=1e-12)


# --------------------------------------------------------------- backward ---

def torch_grads(q, k, v, dout, causal, scale):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).requires_grad_(True) for x in (q, k, v))
    g = qt.shape[1] // kt.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(g, 1), vt.repeat_interleave(g, 1), is_causal=causal, scale=scale)
    o.backward(torch.from_numpy(dout))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,H_kv,N,d", [(1, 2, 2, 64, 32), (2, 4, 2, 23, 8), (1, 4, 1, 17, 16)])
def test_bwd_matches_torch_autograd(B, H, H_kv, N, d, causal):
    q, k, v, do = rand(B, H, N, d), rand(B, H_kv, N, d), rand(B, H_kv, N, d), rand(B, H, N, d)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv, o, lse = orc.attention_bwd(q, k, v, do, causal, scale)
    tq, tk, tv = torch_grads(q, k, v, do, causal, scale)
    np.testing.assert_allclose(dq, tq, atol=1e-12)
    np.testing.assert_allclose(dk, tk, atol=1e-12)
    np.testing.assert_allclose(dv, tv, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_returns_the_forward(causal):
    """attention_bwd also yields O and LSE (one pass computes forward and backward together, the
    fused forward+backward of the MoA paper, section 4.5): pinned to torch SDPA and logsumexp."""
    B, H, H_kv, N, d = 2, 4, 2, 29, 8
    q, k, v, do = rand(B, H, N, d), rand(B, H_kv, N, d), rand(B, H_kv, N, d), rand(B, H, N, d)
    _, _, _, o, lse = orc.attention_bwd(q, k, v, do, causal, 0.4)
    np.testing.assert_allclose(o, sdpa(q, k, v, causal, 0.4), atol=1e-12)
    s = 0.4 * torch.from_numpy(q) @ torch.from_numpy(np.repeat(k, 2, axis=1)).transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (2, 1)])
def test_bwd_finite_differences(causal, H, H_kv):
    N, d, scale, h = 9, 4, 0.7, 1e-6
    q, k, v, do = rand(1, H, N, d), rand(1, H_kv, N, d), rand(1, H_kv, N, d), rand(1, H, N, d)
    dq, dk, dv, _, _ = orc.attention_bwd(q, k, v, do, causal, scale)

    def loss(q_, k_, v_):
        return float(np.sum(orc.attention_fwd(q_, k_, v_, causal, scale)[0] * do))

    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{k_ + "_": a for k_, a in args_p.items()})
                        - loss(**{k_ + "_": a for k_, a in args_m.items()})) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(grad)))
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_sum_invariants(causal):
    N, d = 80, 16
    q, k, v, do = rand(2, 2, N, d), rand(2, 2, N, d), rand(2, 2, N, d), rand(2, 2, N, d)
    dq, dk, dv, o, lse = orc.attention_bwd(q, k, v, do, causal, 0.25)
    # rows of dS sum to zero, so the key gradients sum to zero over keys
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # rows of P sum to one, so the value gradients sum to the upstream gradient
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def test_bwd_constant_v_and_zero_scale():
    N, d = 30, 8
    q, k, do = rand(1, 2, N, d), rand(1, 2, N, d), rand(1, 2, N, d)
    v = np.broadcast_to(rand(d), (1, 2, N, d)).copy()
    dq, dk, dv, _, _ = orc.attention_bwd(q, k, v, do, True, 0.4)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)
    v2 = rand(1, 2, N, d)
    dq, dk, dv, _, _ = orc.attention_bwd(q, k, v2, do, False, 0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv, np.broadcast_to(do.mean(axis=2, keepdims=True), dv.shape) * 1.0, atol=1e-13)


def test_bwd_causal_last_key():
    N, d, scale = 25, 8, 0.35
    q, k, v, do = rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d)
    dq, dk, dv, o, lse = orc.attention_bwd(q, k, v, do, True, scale)
    # only the last query sees the last key: dV_{N-1} = p_{N-1,N-1} dO_{N-1}
    p_last = math.exp(scale * float(q[0, 0, -1] @ k[0, 0, -1]) - lse[0, 0, -1])
    np.testing.assert_allclose(dv[0, 0, -1], p_last * do[0, 0, -1], atol=1e-14)


# ------------------------------------------------------- ragged prefill ---

def packed(lengths, H, H_kv, d):
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return rand(T, H, d), rand(T, H_kv, d), rand(T, H_kv, d), cu


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2), (4, 1)])
def test_varlen_equals_block_diagonal_mask(causal, H, H_kv):
    # A different formulation: one attention over all T packed rows whose mask allows exactly the
    # pairs inside one sequence (and j <= i within it when causal), via torch SDPA in float64.
    lengths = [5, 1, 0, 12, 7]
    q, k, v, cu = packed(lengths, H, H_kv, 8)
    scale = 0.35
    o, lse = orc.attention_fwd_varlen(q, k, v, cu, causal, scale)
    T = q.shape[0]
    seq = np.repeat(np.arange(len(lengths)), lengths)
    pos = np.arange(T)
    allow = seq[:, None] == seq[None, :]
    if causal:
        allow &= pos[None, :] <= pos[:, None]
    g = H // H_kv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None].repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v).permute(1, 0, 2)[None].repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(allow),
                                                           scale=scale)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    s = scale * (qt @ kt.transpose(-1, -2))
    ref_lse = torch.logsumexp(s.masked_fill(~torch.from_numpy(allow), float("-inf")), dim=-1)[0].numpy()
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_varlen_single_sequence_is_dense():
    q, k, v, cu = packed([19], 4, 2, 8)
    o, lse = orc.attention_fwd_varlen(q, k, v, cu, True, 0.5)
    od, ld = orc.attention_fwd(q.transpose(1, 0, 2)[None], k.transpose(1, 0, 2)[None],
                               v.transpose(1, 0, 2)[None], True, 0.5)
    np.testing.assert_allclose(o, od[0].transpose(1, 0, 2), atol=1e-13)
    np.testing.assert_allclose(lse, ld[0], atol=1e-13)


def test_varlen_sequence_order_does_not_matter():
    lengths = [6, 9, 3]
    q, k, v, cu = packed(lengths, 2, 2, 4)
    o, lse = orc.attention_fwd_varlen(q, k, v, cu, True, 0.8)
    order = [2, 0, 1]
    idx = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in order])
    cu2 = np.concatenate([[0], np.cumsum([lengths[b] for b in order])])
    o2, lse2 = orc.attention_fwd_varlen(q[idx], k[idx], v[idx], cu2, True, 0.8)
    np.testing.assert_allclose(o2, o[idx], atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, idx], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_rows_agree_with_full(causal):
    q, k, v, cu = packed([4, 11, 1, 7], 4, 2, 8)
    o, lse = orc.attention_fwd_varlen(q, k, v, cu, causal, 0.3)
    rows = np.array([(0, 0), (3, 1), (4, 3), (14, 2), (15, 0), (22, 3), (16, 1)])
    ro, rl = orc.attention_fwd_varlen_rows(q, k, v, cu, causal, 0.3, rows)
    np.testing.assert_allclose(ro, o[rows[:, 0], rows[:, 1]], atol=1e-13)
    np.testing.assert_allclose(rl, lse[rows[:, 1], rows[:, 0]], atol=1e-13)



@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2), (4, 1)])
def test_varlen_bwd_matches_autograd_with_block_diagonal_mask(causal, H, H_kv):
    # torch autograd in float64 over all T packed rows at once, the sequences kept apart only by an
    # explicit mask (and key <= query within a sequence when causal), KV heads expanded for groups.
    lengths = [5, 1, 0, 12, 7]
    q, k, v, cu = packed(lengths, H, H_kv, 8)
    do = rand(*q.shape)
    scale = 0.35
    dq, dk, dv, o, lse = orc.attention_bwd_varlen(q, k, v, do, cu, causal, scale)
    T = q.shape[0]
    seq = np.repeat(np.arange(len(lengths)), lengths)
    pos = np.arange(T)
    allow = seq[:, None] == seq[None, :]
    if causal:
        allow &= pos[None, :] <= pos[:, None]
    g = H // H_kv
    qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    qh = qt.permute(1, 0, 2)  # [H, T, d]
    kh = kt.permute(1, 0, 2).repeat_interleave(g, dim=0)
    vh = vt.permute(1, 0, 2).repeat_interleave(g, dim=0)
    s = (scale * (qh @ kh.transpose(-1, -2))).masked_fill(~torch.from_numpy(allow), float("-inf"))
    ot = torch.softmax(s, dim=-1) @ vh
    ot.backward(torch.from_numpy(do).permute(1, 0, 2))
    np.testing.assert_allclose(o, ot.detach().permute(1, 0, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).detach().numpy(), atol=1e-12)
    for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(got, ref.numpy(), atol=1e-12)


def test_varlen_bwd_finite_differences():
    # Central differences of L = sum(O * dO) through the (separately pinned) ragged forward, on a
    # batch with an empty sequence and a grouped KV head.
    lengths = [3, 0, 5]
    q, k, v, cu = packed(lengths, 2, 1, 4)
    do = rand(*q.shape)
    scale, h = 0.6, 1e-6
    dq, dk, dv, _, _ = orc.attention_bwd_varlen(q, k, v, do, cu, True, scale)

    def loss(args):
        return float(np.sum(orc.attention_fwd_varlen(args["q"], args["k"], args["v"], cu, True, scale)[0] * do))

    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            num[idx] = (loss({"q": q, "k": k, "v": v, name: xp}) - loss({"q": q, "k": k, "v": v, name: xm})) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(grad)))
        assert err < 1e-7, (name, err)


# ---------------------------------------------------------------- fp8 (E4M3) ---
# The format is OCP FP8 E4M3 (FN variant), the e4m3 of "FP8 Formats for Deep Learning" (listed
# among the sources of "Why Fast GPUs Still Wait for Memory"): bias 7, no infinities, NaN at
# S.1111.111, largest finite 448, subnormals (M / 8) * 2^-6.

ALL_CODES = np.arange(256, dtype=np.uint8)


def torch_e4m3(codes):
    """Library decode: torch's float8_e4m3fn -> float64 upcast (shares nothing with the oracle)."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_matches_torch_on_every_code():
    a, b = orc.e4m3_decode(ALL_CODES), torch_e4m3(ALL_CODES)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])
    assert np.array_equal(np.signbit(a[~np.isnan(a)]), np.signbit(b[~np.isnan(b)]))  # -0 too


def test_e4m3_decode_closed_forms():
    d = orc.e4m3_decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0        # largest finite: 1.75 * 2^8
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9  # subnormals: M * 2^-9
    assert d(0x08) == 2.0 ** -6                         # smallest normal
    assert d(0x38) == 1.0 and d(0x3F) == 1.875 and d(0x40) == 2.0 and d(0xB8) == -1.0
    assert d(0x00) == 0.0 and np.signbit(d(0x80)) and d(0x80) == 0.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x78) == 256.0 and d(0x77) == 240.0        # E = 15 is a finite binade except M = 7
    pos = orc.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)                     # codes 0..126 increase strictly
    assert np.array_equal(orc.e4m3_decode(ALL_CODES[128:255]), -pos)
    # within a binade the 8 steps are equal: 2^(E - 7) / 8
    for e in range(1, 16):
        vals = orc.e4m3_decode(np.array([(e << 3) | m for m in range(7 if e == 15 else 8)], dtype=np.uint8))
        assert np.allclose(np.diff(vals), 2.0 ** (e - 7) / 8, rtol=0, atol=0)


def fp8_case(B, H, H_kv, N, d, seed=0):
    g = np.random.default_rng(seed)
    # finite codes only (0x7F / 0xFF are NaN)
    draw = lambda *s: np.where((c := g.integers(0, 256, size=s, dtype=np.uint8)) & 0x7F == 0x7F, c ^ 1, c).astype(np.uint8)
    return draw(B, H, N, d), draw(B, H_kv, N, d), draw(B, H_kv, N, d)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_fwd_matches_torch_decode_and_sdpa(causal):
    q8, k8, v8 = fp8_case(2, 4, 2, 19, 16)
    # random codes span 2^-9 .. 448; a small scale keeps the softmax from saturating to one-hot
    ds, scale = (0.01, 0.02, 0.5), 0.07
    o, lse = orc.attention_fwd_fp8(q8, k8, v8, ds, causal, scale)
    q, k, v = (f * torch_e4m3(x) for f, x in zip(ds, (q8, k8, v8)))
    np.testing.assert_allclose(o, sdpa(q, k, v, causal, scale), rtol=1e-12, atol=1e-12)
    s = scale * np.einsum("bhid,bhjd->bhij", q, np.repeat(k, 2, axis=1))
    if causal:
        s = np.where(np.tril(np.ones((19, 19), dtype=bool)), s, -np.inf)
    mx = s.max(-1, keepdims=True)
    np.testing.assert_allclose(lse, (mx + np.log(np.exp(s - mx).sum(-1, keepdims=True)))[..., 0], rtol=1e-12)


def test_fp8_descales_enter_as_exact_factors():
    q8, k8, v8 = fp8_case(1, 2, 2, 11, 8, seed=1)
    o1, l1 = orc.attention_fwd_fp8(q8, k8, v8, (0.01, 0.02, 1.0), True, 0.1)
    o2, l2 = orc.attention_fwd_fp8(q8, k8, v8, (0.01, 0.02, 4.0), True, 0.1)   # V descale scales O only
    np.testing.assert_array_equal(o2, 4.0 * o1)
    np.testing.assert_array_equal(l2, l1)
    o3, l3 = orc.attention_fwd_fp8(q8, k8, v8, (0.02, 0.01, 1.0), True, 0.1)   # only dq * dk matters
    np.testing.assert_allclose(o3, o1, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l3, l1, rtol=1e-14)
    o4, l4 = orc.attention_fwd_fp8(q8, k8, v8, (0.01, 0.04, 1.0), True, 0.05)  # ... times the scale
    np.testing.assert_allclose(o4, o1, rtol=1e-14, atol=1e-14)


def test_fp8_rows_agree_with_full():
    q8, k8, v8 = fp8_case(2, 4, 1, 13, 8, seed=2)
    ds = (0.03, 0.01, 0.25)
    o, lse = orc.attention_fwd_fp8(q8, k8, v8, ds, True, 0.2)
    rows = np.array([(0, 0, 0), (1, 3, 12), (0, 2, 5), (1, 1, 7)])
    ro, rl = orc.attention_fwd_fp8_rows(q8, k8, v8, ds, True, 0.2, rows)
    np.testing.assert_allclose(ro, o[rows[:, 0], rows[:, 1], rows[:, 2]], atol=1e-13)
    np.testing.assert_allclose(rl, lse[rows[:, 0], rows[:, 1], rows[:, 2]], atol=1e-13)
