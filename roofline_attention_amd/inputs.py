"""Seeded synthetic inputs for the attention path and its oracle.

This module is shared by the HIP path's tests/benchmark and by the oracle's
checks. It holds no attention arithmetic: it only draws random numbers, rounds
them to the storage dtype and lays them out.

Recipe (the pages fix none of it; the workloads are synthetic sweeps shaped like
"Why Fast GPUs Still Wait for Memory", section "Attention from first principles"
(N = 4096, d = 128, bf16) and the MoA paper's section 2.2 (B = 2, D = 64)):

* every (tensor, batch, head) block is drawn from its own numpy stream,
  ``Generator(PCG64(SeedSequence([seed, tensor_id, b, h])))``, as
  ``standard_normal(shape, dtype=float32)``; a per-block stream lets a checker
  regenerate one head of a large tensor without drawing the rest;
* tensor ids: q = 0, k = 1, v = 2, dO = 3, kv_len = 4;
* an optional exact factor (0.5 for the large prefill workload) multiplies the
  float32 sample before rounding;
* bf16 storage uses round-to-nearest-even (torch's float32 -> bfloat16 cast);
* decode KV lengths are integers drawn inclusively from [lo, hi]; cache rows at
  or beyond a sequence's length are filled with NaN so that any read of them
  shows up in the result;
* a ragged prefill batch draws its lengths from the same length stream and packs
  the (b, h) blocks of each tensor row after row ([T, H, d], offsets cu_seqlens);
* fp8 (E4M3) storage: each tensor's float32 sample is divided by a per-tensor
  power-of-two descale, the smallest with amax / descale <= 448 (so the division
  is exact and nothing saturates), and rounded to nearest even by torch's
  float32 -> float8_e4m3fn cast; the codes are kept as uint8 and the descale is
  handed to both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO, TENSOR_KVLEN = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """One frozen case: operation, shape, dtype, mask and seed."""

    name: str
    op: str  # "fwd", "decode" or "fwdbwd"
    B: int
    H: int
    H_kv: int
    N: int  # sequence length (prefill) or cache capacity (decode)
    d: int
    dtype: str  # "f32", "bf16" or "e4m3"
    causal: bool
    seed: int
    qk_factor: float = 1.0  # exact factor applied to Q and K samples
    kv_lo: int = 0  # decode only: inclusive KV-length range
    kv_hi: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads of the headline metric, then the ragged prefill.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "fwd", 1, 2, 2, 128, 64, "f32", False, seed=1),
    "prefill_causal_1k": Workload("prefill_causal_1k", "fwd", 4, 16, 16, 1024, 64, "bf16", True, seed=2),
    "prefill_4k_causal": Workload("prefill_4k_causal", "fwd", 2, 32, 32, 4096, 128, "bf16", True, seed=3,
                                  qk_factor=0.5),
    "prefill_4k": Workload("prefill_4k", "fwd", 2, 32, 32, 4096, 128, "bf16", False, seed=3, qk_factor=0.5),
    "decode_gqa": Workload("decode_gqa", "decode", 64, 32, 8, 8192, 128, "bf16", False, seed=4,
                           kv_lo=512, kv_hi=8192),
    "fwdbwd_4k_causal": Workload("fwdbwd_4k_causal", "fwdbwd", 2, 16, 16, 4096, 128, "bf16", True, seed=5),
    # Ragged prefill (packed rows, per-sequence offsets): 16 sequences with the decode length mix,
    # grouped heads 32/8; N is the longest length the grid must cover.
    # The large prefill with fp8 (E4M3) inputs and per-tensor descales.
    "prefill_4k_causal_fp8": Workload("prefill_4k_causal_fp8", "fwd", 2, 32, 32, 4096, 128, "e4m3", True, seed=7,
                                      qk_factor=0.5),
    "prefill_4k_fp8": Workload("prefill_4k_fp8", "fwd", 2, 32, 32, 4096, 128, "e4m3", False, seed=7, qk_factor=0.5),
    "prefill_varlen": Workload("prefill_varlen", "varlen", 16, 32, 8, 8192, 128, "bf16", True, seed=6,
                               kv_lo=512, kv_hi=8192),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def normal_block(seed: int, tensor_id: int, b: int, h: int, shape, factor: float = 1.0) -> np.ndarray:
    """float32 N(0,1) sample for one (tensor, batch, head) block."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, b, h])))
    x = g.standard_normal(shape, dtype=np.float32)
    if factor != 1.0:
        x *= np.float32(factor)  # 0.5 is exact in float32
    return x


def make_tensor(seed: int, tensor_id: int, B: int, H: int, rows: int, d: int, dtype: str,
                factor: float = 1.0) -> torch.Tensor:
    """[B, H, rows, d] CPU tensor in the storage dtype, one stream per (b, h)."""
    out = torch.empty((B, H, rows, d), dtype=torch_dtype(dtype))
    for b in range(B):
        for h in range(H):
            blk = torch.from_numpy(normal_block(seed, tensor_id, b, h, (rows, d), factor))
            out[b, h].copy_(blk)  # float32 -> bf16 cast rounds to nearest even
    return out


def fp8_codes(x: torch.Tensor):
    """(uint8 E4M3 codes, descale) for a float32 tensor, with a power-of-two descale."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    descale = 2.0 ** math.ceil(math.log2(amax / 448.0)) if amax > 0 else 1.0
    codes = (x / descale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, descale


def make_fp8_prefill(w: Workload) -> dict:
    """q, k, v as uint8 E4M3 codes [B,H,N,d] / [B,H_kv,N,d] and descale = (dq, dk, dv)."""
    out, ds = {}, []
    for name, tid, heads, f in (("q", TENSOR_Q, w.H, w.qk_factor), ("k", TENSOR_K, w.H_kv, w.qk_factor),
                                ("v", TENSOR_V, w.H_kv, 1.0)):
        x = make_tensor(w.seed, tid, w.B, heads, w.N, w.d, "f32", f)
        out[name], s = fp8_codes(x)
        ds.append(s)
    out["descale"] = tuple(ds)
    return out


def kv_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TENSOR_KVLEN])))
    return g.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def make_prefill(w: Workload, with_dout: Optional[bool] = None) -> dict:
    """q, k, v (and dO for fwd+bwd) as CPU tensors in the storage dtype."""
    if with_dout is None:
        with_dout = w.op == "fwdbwd"
    t = {
        "q": make_tensor(w.seed, TENSOR_Q, w.B, w.H, w.N, w.d, w.dtype, w.qk_factor),
        "k": make_tensor(w.seed, TENSOR_K, w.B, w.H_kv, w.N, w.d, w.dtype, w.qk_factor),
        "v": make_tensor(w.seed, TENSOR_V, w.B, w.H_kv, w.N, w.d, w.dtype),
    }
    if with_dout:
        t["do"] = make_tensor(w.seed, TENSOR_DO, w.B, w.H, w.N, w.d, w.dtype)
    return t


def make_varlen(w: Workload, lengths=None, with_dout: bool = False) -> dict:
    """Packed ragged batch: q [T,H,d], k/v [T,H_kv,d], cu_seqlens [B+1] int32, lengths [B], and
    with_dout an upstream gradient "do" [T,H,d].

    Lengths come from the kv-length stream (inclusive [kv_lo, kv_hi]) unless given; the rows of
    sequence b and head h are the (b, h) block of each tensor's streams, placed at rows
    cu_seqlens[b] .. cu_seqlens[b+1] - 1.
    """
    if lengths is None:
        lengths = kv_lengths(w.seed, w.B, w.kv_lo, w.kv_hi)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    dt = torch_dtype(w.dtype)
    out = {}
    for name, tid, heads, factor in (("q", TENSOR_Q, w.H, w.qk_factor), ("k", TENSOR_K, w.H_kv, w.qk_factor),
                                     ("v", TENSOR_V, w.H_kv, 1.0), ("do", TENSOR_DO, w.H, 1.0)):
        if name == "do" and not with_dout:
            continue
        t = torch.empty((T, heads, w.d), dtype=dt)
        for b in range(len(lengths)):
            for h in range(heads):
                blk = normal_block(w.seed, tid, b, h, (int(lengths[b]), w.d), factor)
                t[cu[b]:cu[b + 1], h].copy_(torch.from_numpy(blk))
        out[name] = t
    out["cu_seqlens"] = torch.from_numpy(cu)
    out["lengths"] = lengths
    return out


def make_decode(w: Workload, nan_pad: bool = True) -> dict:
    """q [B, H, d]; k/v caches [B, H_kv, N_cap, d]; kv_len [B] int32."""
    kv_len = kv_lengths(w.seed, w.B, w.kv_lo, w.kv_hi)
    q = make_tensor(w.seed, TENSOR_Q, w.B, w.H, 1, w.d, w.dtype, w.qk_factor)[:, :, 0, :].contiguous()
    k = make_tensor(w.seed, TENSOR_K, w.B, w.H_kv, w.N, w.d, w.dtype, w.qk_factor)
    v = make_tensor(w.seed, TENSOR_V, w.B, w.H_kv, w.N, w.d, w.dtype)
    if nan_pad:
        for b in range(w.B):
            k[b, :, int(kv_len[b]):, :] = float("nan")
            v[b, :, int(kv_len[b]):, :] = float("nan")
    return {"q": q, "k": k, "v": v, "kv_len": torch.from_numpy(kv_len)}


def make_decode_paged(w: Workload, page_size: int, dense: Optional[dict] = None, spare_pages: int = 3) -> dict:
    """The decode workload's caches cut into pages [P, H_kv, page_size, d] at shuffled physical slots.

    Sequence b uses ceil(kv_len[b] / page_size) pages; the physical order is a seeded permutation,
    `spare_pages` unreferenced NaN pages sit among them, rows past kv_len in a last page are NaN, and
    unused block-table entries are -1. Returns q, k_pages, v_pages, block_table [B, max_pages],
    kv_len (the same q and rows as make_decode).
    """
    if dense is None:
        dense = make_decode(w)
    kv_len = dense["kv_len"].numpy()
    max_pages = (w.N + page_size - 1) // page_size
    n_pages = [(int(n) + page_size - 1) // page_size for n in kv_len]
    P = sum(n_pages) + spare_pages
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, TENSOR_KVLEN, page_size])))
    slots = g.permutation(P)
    dt = dense["k"].dtype
    kp = torch.full((P, w.H_kv, page_size, w.d), float("nan"), dtype=dt)
    vp = torch.full((P, w.H_kv, page_size, w.d), float("nan"), dtype=dt)
    table = torch.full((w.B, max_pages), -1, dtype=torch.int32)
    nxt = 0
    for b in range(w.B):
        for j in range(n_pages[b]):
            phys = int(slots[nxt])
            nxt += 1
            r0, r1 = j * page_size, min((j + 1) * page_size, w.N)
            kp[phys, :, :r1 - r0] = dense["k"][b, :, r0:r1]
            vp[phys, :, :r1 - r0] = dense["v"][b, :, r0:r1]
            table[b, j] = phys
    return {"q": dense["q"], "k_pages": kp, "v_pages": vp, "block_table": table, "kv_len": dense["kv_len"]}


def decode_head_slices(w: Workload, b: int, hk: int, length: int):
    """Regenerate the first `length` rows of one KV head of a decode cache (no NaN pad)."""
    rows = w.N
    k = torch.from_numpy(normal_block(w.seed, TENSOR_K, b, hk, (rows, w.d), w.qk_factor)[:length])
    v = torch.from_numpy(normal_block(w.seed, TENSOR_V, b, hk, (rows, w.d))[:length])
    return k.to(torch_dtype(w.dtype)), v.to(torch_dtype(w.dtype))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of stored values for the fp64 oracle."""
    return t.detach().to("cpu", torch.float64).numpy()
