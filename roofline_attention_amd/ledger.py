"""Analytic work and byte ledger for the attention path, and the MI355X roofline denominators.

Formulas ("Why Fast GPUs Still Wait for Memory"):
  * FLOPs count an FMA as two operations (section "Compute time, and why peak lies");
  * attention forward W = 4 N^2 d per head (section "Attention from first principles"), halved
    under a causal mask (note "causal masking is not an optimisation here");
  * compulsory bytes: every input crosses HBM once and every output is written once (section
    "The compulsory bound", Q = 4 s N d per head for the forward);
  * naive attention intensity N d / [s (N + d)] (section "Attention from first principles"),
    tiled FlashAttention-2 intensity 4N^2d / [s(2Nd + 2N^2 d / B_r)] (section "The tiled bound");
  * decode W = 4 N d, Q = 2 s N d per KV head and I = 2g/s under grouped queries (section
    "Attention III - KV cache, GQA, MLA").
The backward counts the five N^2 d products a non-materialising backward needs (S recompute, dP,
dV, dK, dQ): W_bwd = 2.5 W_fwd. Recompute beyond those is implementation cost, not work.

MI355X peaks (AMD's published figures, not on the pages): dense bf16 MFMA 2516.6 TFLOP/s
(256 CU x 2.4 GHz x 4096 FLOP/clk/CU), dense fp8 MFMA 5033.2 TFLOP/s (twice bf16, as the pages
say of fp8 in general: section "pi is the top of a stack", Table 1), HBM3E 8.0 TB/s.
"""
from __future__ import annotations

PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 5033.2
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def fwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    w = 4.0 * B * H * N * N * d
    return w / 2 if causal else w


def varlen_fwd_flops(H: int, d: int, lengths, causal: bool) -> float:
    """Algorithmic forward FLOPs of a ragged batch: each sequence counts as its own dense case."""
    return sum(fwd_flops(1, H, int(n), d, causal) for n in lengths)


def bwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    return 2.5 * fwd_flops(B, H, N, d, causal)


def fwd_bytes(B: int, H: int, H_kv: int, N: int, d: int, s: int, lse: bool = True) -> float:
    """Compulsory HBM bytes of the forward: read Q, K, V once, write O (and fp32 LSE) once."""
    b = s * N * d * (2 * B * H + 2 * B * H_kv)
    return b + (4.0 * B * H * N if lse else 0.0)


def bwd_bytes(B: int, H: int, H_kv: int, N: int, d: int, s: int, grad_bytes: int = 4) -> float:
    """Compulsory bytes of the backward: read Q, K, V, O, dO and LSE; write dQ, dK, dV."""
    reads = s * N * d * (3 * B * H + 2 * B * H_kv) + 4.0 * B * H * N
    writes = grad_bytes * N * d * (B * H + 2 * B * H_kv)
    return reads + writes


def decode_flops(H: int, d: int, kv_lens) -> float:
    return 4.0 * d * H * float(sum(int(x) for x in kv_lens))


def decode_bytes(H: int, H_kv: int, d: int, s: int, kv_lens, lse: bool = True) -> float:
    """Compulsory bytes of decode: the valid K and V rows once, q read once, o (and lse) written once."""
    B = len(kv_lens)
    kv = 2.0 * s * d * H_kv * float(sum(int(x) for x in kv_lens))
    return kv + 2.0 * s * B * H * d + (4.0 * B * H if lse else 0.0)


def naive_intensity(N: int, d: int, s: int) -> float:
    return N * d / (s * (N + d))


def compulsory_intensity(N: int, s: int) -> float:
    return N / s


def tiled_intensity(N: int, d: int, s: int, B_r: int) -> float:
    return 4.0 * N * N * d / (s * (2.0 * N * d + 2.0 * N * N * d / B_r))


def decode_intensity(g: int, s: int) -> float:
    return 2.0 * g / s


def round_trip_bytes(M: int, N: int, s: int) -> float:
    """Bytes a fused kernel removes by not writing and re-reading an M x N intermediate
    ("M4.2 - GPU Execution Model for Transformer Kernels", section 0x08 fusion ledger)."""
    return 2.0 * M * N * s


def moa_naive_fwd_bytes(B: int, N: int, D: int, s: int = 8):
    """Bytes of the MoA paper's naive forward (reads Q, K, V; writes the n x n matrix A and Out)."""
    reads = 3.0 * B * N * D * s
    writes = B * N * N * s + B * N * D * s
    return reads, writes, reads + writes
