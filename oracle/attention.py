"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never calls it, and this module imports nothing from the
product package.

What it computes is the plain definition, with the score matrix materialised:
"Why Fast GPUs Still Wait for Memory", section "Attention from first
principles": S = Q K^T, P = softmax(S) row by row, O = P V. The same page,
section "FlashAttention is an IO algorithm", states that the tiled online-softmax
schedule changes only the memory traffic, not the arithmetic result, so the
naive schedule written here is the exact reference for the fused kernels.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * the score carries a caller-given factor: S = scale * Q K^T (the pages write
    S = Q K^T; the configured workloads use scale = 1/sqrt(d));
  * causal keeps the lower triangle including the diagonal (key j <= query i),
    following the page's "Nuance - causal masking" note, with N_q = N_k;
  * grouped-query attention maps query head h to KV head h // (H / H_kv)
    (section "Attention III - KV cache, GQA, MLA" gives only g = h / h_kv);
  * LSE is the natural-log log-sum-exp of each score row over unmasked keys;
  * decode is one query row against the first kv_len[b] cache rows; a paged cache
    maps logical row j to row j % page_size of page block_table[b, j // page_size];
  * a ragged (variable-length) batch packs its sequences' rows one after another
    ([T, H, d], offsets cu_seqlens); each sequence attends only within itself, and a
    causal position is counted from the sequence's first row;
  * fp8 inputs are OCP FP8 E4M3 codes (the "FN" variant: exponent bias 7, no
    infinities, S.1111.111 is NaN, largest finite value 448), the e4m3 format of
    "FP8 Formats for Deep Learning" (in the same page's sources), with one
    float32 descale factor per tensor (real value = descale * decoded code); the
    result is exact attention of those real values ("Why Fast GPUs Still Wait for
    Memory" names fp8 only through its doubled compute ceiling, section "pi is the
    top of a stack" and Table 1, and leaves the format and its scaling metadata open);
  * the backward pass is the gradient of L = sum(O * dO) with respect to Q, K
    and V, recomputing P from an explicit S (same page: "the backward pass does
    more arithmetic, because S is recomputed rather than stored"; the MoA paper,
    section 4.1, computes GQ, GK, GV the same way from Q, K, V).

All arithmetic is in float64 numpy. Matrix products use numpy's matmul as the
library primitive for a contraction; there is no tiling or reordering beyond
the definition. Every function returns new arrays and keeps no state.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np


def _check_shapes(q, k, v):
    B, H, N, d = q.shape
    Bk, H_kv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if H % H_kv != 0:
        raise ValueError("H must be a multiple of H_kv")
    return B, H, H_kv, N, d


def _scores(qh: np.ndarray, kh: np.ndarray, causal: bool, scale: float) -> np.ndarray:
    """Explicit score matrix S = scale * q k^T, masked entries set to -inf."""
    s = scale * (qh @ kh.T)
    if causal:
        n_q, n_k = s.shape
        above = np.triu(np.ones((n_q, n_k), dtype=bool), k=1)  # key j > query i
        s[above] = -np.inf
    return s


def _softmax_rows(s: np.ndarray):
    """Row softmax with the row maximum subtracted first; also returns ln-sum-exp."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    lse = (m + np.log(l))[:, 0]
    return p, lse


def attention_fwd(q, k, v, causal: bool, scale: float):
    """O [B,H,N,d] and LSE [B,H,N] for q [B,H,N,d], k/v [B,H_kv,N,d] (float64)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, H_kv, N, d = _check_shapes(q, k, v)
    g = H // H_kv
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            hk = h // g
            s = _scores(q[b, h], k[b, hk], causal, scale)
            p, lse[b, h] = _softmax_rows(s)
            o[b, h] = p @ v[b, hk]
    return o, lse


def attention_fwd_rows(q, k, v, causal: bool, scale: float, rows):
    """O and LSE for selected (b, h, i) query rows only, each from its own score row.

    rows: integer array [n, 3] of (b, h, i). Returns (o [n, d], lse [n]).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, H_kv, N, d = _check_shapes(q, k, v)
    g = H // H_kv
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    o = np.empty((len(rows), d))
    lse = np.empty(len(rows))
    for r, (b, h, i) in enumerate(rows):
        hk = h // g
        n_keys = i + 1 if causal else N  # causal row i sees keys 0..i
        s = scale * (k[b, hk, :n_keys] @ q[b, h, i])
        p, lse_r = _softmax_rows(s[None, :])
        o[r] = p[0] @ v[b, hk, :n_keys]
        lse[r] = lse_r[0]
    return o, lse


def attention_fwd_varlen(q, k, v, cu_seqlens, causal: bool, scale: float):
    """Variable-length (ragged) prefill over packed token rows.

    q [T, H, d], k/v [T, H_kv, d]; sequence b owns rows cu_seqlens[b] .. cu_seqlens[b+1] - 1
    and attends only within itself, with positions counted from its own first row (causal:
    key j <= query i within the sequence). Returns o [T, H, d] and lse [H, T]. The definition of
    "Attention from first principles" is applied to each sequence on its own: a ragged batch is
    a set of independent sequences addressed by per-sequence offsets.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    T, H, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (T, H_kv, d) or v.shape != k.shape or H % H_kv != 0:
        raise ValueError("expected q [T,H,d], k/v [T,H_kv,d] with H % H_kv == 0")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at T and not decrease")
    g = H // H_kv
    o = np.zeros((T, H, d))
    lse = np.zeros((H, T))
    for b in range(len(cu) - 1):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 == r0:
            continue
        for h in range(H):
            hk = h // g
            s = _scores(q[r0:r1, h], k[r0:r1, hk], causal, scale)
            p, lse[h, r0:r1] = _softmax_rows(s)
            o[r0:r1, h] = p @ v[r0:r1, hk]
    return o, lse


def attention_fwd_varlen_rows(q, k, v, cu_seqlens, causal: bool, scale: float, rows):
    """O and LSE of selected (token, head) rows of the ragged prefill, each from its own score row.

    rows: integer array [n, 2] of (t, h). Returns (o [n, d], lse [n]).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    H, H_kv, d = q.shape[1], k.shape[1], q.shape[2]
    g = H // H_kv
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    o = np.empty((len(rows), d))
    lse = np.empty(len(rows))
    for r, (t, h) in enumerate(rows):
        b = int(np.searchsorted(cu, t, side="right")) - 1  # cu[b] <= t < cu[b+1]
        r0, r1 = int(cu[b]), int(cu[b + 1])
        hk = h // g
        k_end = t + 1 if causal else r1  # causal row t sees the sequence's rows r0 .. t
        s = scale * (k[r0:k_end, hk] @ q[t, h])
        p, lse_r = _softmax_rows(s[None, :])
        o[r] = p[0] @ v[r0:k_end, hk]
        lse[r] = lse_r[0]
    return o, lse


def e4m3_decode(codes) -> np.ndarray:
    """Real values (float64) of OCP FP8 E4M3 codes given as uint8.

    Bit layout S.EEEE.MMM, exponent bias 7: E = 0 is subnormal, (-1)^S * (M / 8) * 2^-6;
    otherwise (-1)^S * (1 + M / 8) * 2^(E - 7), except E = 15 with M = 7, which is NaN
    (the FN variant has no infinities, so its largest finite value is 1.75 * 2^8 = 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >= 128, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def _fp8_real(q8, k8, v8, descale):
    dq, dk, dv = (float(x) for x in descale)
    return dq * e4m3_decode(q8), dk * e4m3_decode(k8), dv * e4m3_decode(v8)


def attention_fwd_fp8(q8, k8, v8, descale, causal: bool, scale: float):
    """Exact attention of fp8 (E4M3) inputs: O [B,H,N,d] and LSE [B,H,N] in float64.

    q8 [B,H,N,d], k8/v8 [B,H_kv,N,d] are uint8 E4M3 codes and descale = (dq, dk, dv) the
    per-tensor factors, so the real inputs are dq * decode(q8), and so on. The attention of
    those real values is the plain definition, computed by attention_fwd.
    """
    q, k, v = _fp8_real(q8, k8, v8, descale)
    return attention_fwd(q, k, v, causal, scale)


def attention_fwd_fp8_rows(q8, k8, v8, descale, causal: bool, scale: float, rows):
    """attention_fwd_rows of the real values of fp8 inputs, for selected (b, h, i) rows."""
    q, k, v = _fp8_real(q8, k8, v8, descale)
    return attention_fwd_rows(q, k, v, causal, scale, rows)


def attention_decode(q, k_cache, v_cache, kv_len, scale: float):
    """One query per (sequence, head) over its first kv_len[b] cached keys.

    q [B,H,d]; k_cache/v_cache [B,H_kv,N_cap,d]; kv_len [B] ints in [1, N_cap].
    Returns (o [B,H,d], lse [B,H]). Cache rows at or beyond kv_len[b] are not read.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, d = q.shape
    H_kv = k_cache.shape[1]
    g = H // H_kv
    o = np.empty((B, H, d))
    lse = np.empty((B, H))
    for b in range(B):
        n = int(kv_len[b])
        if not 1 <= n <= k_cache.shape[2]:
            raise ValueError("kv_len out of range")
        for h in range(H):
            hk = h // g
            kh = np.asarray(k_cache[b, hk, :n], dtype=np.float64)
            vh = np.asarray(v_cache[b, hk, :n], dtype=np.float64)
            s = scale * (kh @ q[b, h])
            p, lse_r = _softmax_rows(s[None, :])
            o[b, h] = p[0] @ vh
            lse[b, h] = lse_r[0]
    return o, lse


def attention_decode_paged(q, k_pages, v_pages, block_table, kv_len, scale: float):
    """Decode over a paged KV cache.

    k_pages/v_pages [P, H_kv, page_size, d] hold the cache in fixed-size pages; logical cache row j
    of sequence b is row j % page_size of physical page block_table[b, j // page_size]. The pages
    of a sequence need not be contiguous or in order ("M4.2 - GPU Execution Model for Transformer
    Kernels", section 0x0D, failure 16: logical K/V continuity does not imply contiguous physical
    addresses). The logical rows are gathered, then the plain decode definition applies.
    Returns (o [B,H,d], lse [B,H]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, d = q.shape
    P, H_kv, ps, _ = k_pages.shape
    g = H // H_kv
    table = np.asarray(block_table, dtype=np.int64)
    o = np.empty((B, H, d))
    lse = np.empty((B, H))
    for b in range(B):
        n = int(kv_len[b])
        if not 1 <= n <= table.shape[1] * ps:
            raise ValueError("kv_len out of range")
        pages = table[b, :(n + ps - 1) // ps]
        for h in range(H):
            hk = h // g
            kh = np.concatenate([np.asarray(k_pages[p, hk], dtype=np.float64) for p in pages])[:n]
            vh = np.concatenate([np.asarray(v_pages[p, hk], dtype=np.float64) for p in pages])[:n]
            s = scale * (kh @ q[b, h])
            pr, lse_r = _softmax_rows(s[None, :])
            o[b, h] = pr[0] @ vh
            lse[b, h] = lse_r[0]
    return o, lse


def attention_bwd(q, k, v, dout, causal: bool, scale: float):
    """Gradients of L = sum(O * dO) for O = softmax(scale Q K^T [mask]) V.

    Returns (dq [B,H,N,d], dk [B,H_kv,N,d], dv [B,H_kv,N,d], o, lse). Under grouped
    heads, dK and dV of a KV head sum the contributions of its query heads.
    Steps, per (b, h), with P recomputed from the explicit S:
        dV += P^T dO
        dP  = dO V^T
        D_i = sum_t dO[i,t] O[i,t]          (= sum_j P_ij dP_ij)
        dS  = P * (dP - D)                   (zero where masked, since P is zero)
        dQ  = scale * dS K
        dK += scale * dS^T Q
    """
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, H, H_kv, N, d = _check_shapes(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    g = H // H_kv
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.empty_like(q)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            hk = h // g
            s = _scores(q[b, h], k[b, hk], causal, scale)
            p, lse[b, h] = _softmax_rows(s)
            o[b, h] = p @ v[b, hk]
            dv[b, hk] += p.T @ dout[b, h]
            dp = dout[b, h] @ v[b, hk].T
            D = np.sum(dout[b, h] * o[b, h], axis=1, keepdims=True)
            ds = p * (dp - D)
            dq[b, h] = scale * (ds @ k[b, hk])
            dk[b, hk] += scale * (ds.T @ q[b, h])
    return dq, dk, dv, o, lse


def attention_bwd_varlen(q, k, v, dout, cu_seqlens, causal: bool, scale: float):
    """Gradients of L = sum(O * dO) for the ragged prefill of attention_fwd_varlen.

    q, dout [T, H, d], k/v [T, H_kv, d], cu_seqlens as in attention_fwd_varlen. Returns
    (dq [T, H, d], dk [T, H_kv, d], dv [T, H_kv, d], o [T, H, d], lse [H, T]). Sequences share
    no score, so each sequence's gradients are the steps of attention_bwd taken on its own rows
    r0 .. r1 - 1 of every head, with causal positions counted from r0.
    """
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    T, H, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (T, H_kv, d) or v.shape != k.shape or dout.shape != q.shape or H % H_kv != 0:
        raise ValueError("expected q, dout [T,H,d], k/v [T,H_kv,d] with H % H_kv == 0")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at T and not decrease")
    g = H // H_kv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros_like(q)
    lse = np.zeros((H, T))
    for b in range(len(cu) - 1):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 == r0:
            continue
        for h in range(H):
            hk = h // g
            qs, ks, vs, dos = q[r0:r1, h], k[r0:r1, hk], v[r0:r1, hk], dout[r0:r1, h]
            p, lse[h, r0:r1] = _softmax_rows(_scores(qs, ks, causal, scale))
            os_ = p @ vs
            o[r0:r1, h] = os_
            dv[r0:r1, hk] += p.T @ dos
            dp = dos @ vs.T
            ds = p * (dp - np.sum(dos * os_, axis=1, keepdims=True))
            dq[r0:r1, h] = scale * (ds @ ks)
            dk[r0:r1, hk] += scale * (ds.T @ qs)
    return dq, dk, dv, o, lse
