"""Python binding of libroofattn.so (ctypes): argument marshalling only.

Every function here checks tensor placement, dtype, contiguity and shape, allocates any output
the caller did not pass (torch is used for device memory and streams only), and calls the C ABI
declared in include/attn.h on torch's current HIP stream. All arithmetic happens in the library's
kernels; there is no fallback path: if the library is missing this module fails to import.
"""
from __future__ import annotations

import atexit
import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ROOFATTN_LIB may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("ROOFATTN_LIB", os.path.join(_HERE, "libroofattn.so"))

ATTN_F32, ATTN_BF16 = 0, 1
# The ABI version these signatures describe (attn_abi_version() of the matching library).
ABI_VERSION = 7
_DTYPES = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}

# Every symbol include/attn.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
SIGNATURES = {
    "attn_abi_version": (_I, []),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P]),
    "attn_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_decode_workspace_size": (_Z, [_I, _I, _I, _I]),
    "attn_decode": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]),
    "attn_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]),
    "attn_bwd_workspace_size": (_Z, [_I, _I, _I, _I]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]),
    "attn_bwd_varlen_workspace_size": (_Z, [_I, _I, _I]),
    "attn_bwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z,
                             _P]),
    "attn_fwd_bwd_workspace_size": (_Z, [_I, _I, _I, _I]),
    "attn_fwd_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]),
    "attn_timing_enable": (_I, [_I]),
    "attn_timing_reset": (_I, []),
    "attn_timing_count": (_I, []),
    "attn_timing_get": (_I, [_I, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_longlong),
                             ctypes.POINTER(ctypes.c_double)]),
    "attn_timing_samples": (_I, [_I, ctypes.POINTER(ctypes.c_float), _I]),
    "attn_release": (_I, []),
}


class AttnError(RuntimeError):
    """A non-zero attn_status returned by the library."""


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m roofline_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.attn_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} reports ABI version {lib.attn_abi_version()}, this binding expects "
                          f"{ABI_VERSION}: rebuild the library from these sources")
    return lib


_lib = load_library()


def release() -> None:
    """Destroys the library's timing events (attn_release); the library stays usable."""
    _check(_lib.attn_release())


# Python's exit handlers run before the C runtime's teardown (and before a profiler attached to the
# process finalises), so no library-owned HIP object is left for that teardown.
atexit.register(lambda: _lib.attn_release())


def abi_version() -> int:
    return _lib.attn_abi_version()


def _check(status: int) -> None:
    if status != 0:
        msg = _lib.attn_last_error().decode()
        raise AttnError(f"{_lib.attn_status_string(status).decode()}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool, scale: Optional[float] = None,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, want_lse: bool = True):
    """Attention forward. q [B,H,N,d], k/v [B,H_kv,N,d] (float32 or bfloat16). Returns (o, lse)."""
    _need(q, "q")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if q.dtype not in _DTYPES:
        raise ValueError("dtype must be float32 or bfloat16")
    _need(k, "k", q.dtype, (B, H_kv, N, d), q.device)
    _need(v, "v", q.dtype, (B, H_kv, N, d), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, q.shape, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H, N), q.device)
    _check(_lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, H_kv, N, d, int(bool(causal)),
                         float(scale), _DTYPES[q.dtype], _stream(q.device)))
    return out, lse


def fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, descale, causal: bool, scale: Optional[float] = None,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, want_lse: bool = True):
    """fp8 forward: q [B,H,N,d], k/v [B,H_kv,N,d] uint8 E4M3 codes, descale = (q, k, v) float factors.

    Returns (o bf16 [B,H,N,d], lse float32 [B,H,N] or None).
    """
    _need(q, "q", torch.uint8)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    _need(k, "k", torch.uint8, (B, H_kv, N, d), q.device)
    _need(v, "v", torch.uint8, (B, H_kv, N, d), q.device)
    dq, dk, dv = (float(x) for x in descale)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, H, N, d), q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H, N), q.device)
    _check(_lib.attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, H_kv, N, d, int(bool(causal)),
                             float(scale), dq, dk, dv, _stream(q.device)))
    return out, lse


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
               causal: bool, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, want_lse: bool = True):
    """Ragged prefill: q [T,H,d], k/v [T,H_kv,d] bf16 packed rows, cu_seqlens [B+1] int32 on the GPU.

    Returns (o [T,H,d], lse [H,T])."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q, k, v must be 3-D [T, H, d]")
    T, H, d = q.shape
    H_kv = k.shape[1]
    _need(k, "k", torch.bfloat16, (T, H_kv, d), q.device)
    _need(v, "v", torch.bfloat16, (T, H_kv, d), q.device)
    _need(cu_seqlens, "cu_seqlens", torch.int32, None, q.device)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with B + 1 >= 2 entries")
    B = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, q.shape, q.device)
    if lse is None and want_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (H, T), q.device)
    _check(_lib.attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), B,
                                int(max_seqlen), T, H, H_kv, d, int(bool(causal)), float(scale), ATTN_BF16,
                                _stream(q.device)))
    return out, lse


def decode_workspace_size(B: int, H: int, N_cap: int, d: int) -> int:
    return int(_lib.attn_decode_workspace_size(B, H, N_cap, d))


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_len: torch.Tensor,
           scale: Optional[float] = None, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, want_lse: bool = True):
    """Decode: q [B,H,d] bf16, caches [B,H_kv,N_cap,d] bf16, kv_len [B] int32 on the GPU. Returns (o, lse)."""
    _need(q, "q", torch.bfloat16)
    B, H, d = q.shape
    H_kv, N_cap = k_cache.shape[1], k_cache.shape[2]
    _need(k_cache, "k_cache", torch.bfloat16, (B, H_kv, N_cap, d), q.device)
    _need(v_cache, "v_cache", torch.bfloat16, (B, H_kv, N_cap, d), q.device)
    _need(kv_len, "kv_len", torch.int32, (B,), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, q.shape, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H), q.device)
    need = decode_workspace_size(B, H, N_cap, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(_lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _ptr(kv_len), B, H, H_kv,
                            N_cap, d, 0, float(scale), ATTN_BF16, _ptr(workspace), workspace.numel(),
                            _stream(q.device)))
    return out, lse


DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20  # ATTN_DECODE_NOALLOC_SCRATCH_BYTES


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_len: torch.Tensor,
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None):
    """decode() on the library's fixed scratch (attn_decode_noalloc): no workspace, no allocation in
    the library. Outputs the caller does not pass are allocated here by torch. Returns (o, lse)."""
    _need(q, "q", torch.bfloat16)
    B, H, d = q.shape
    H_kv, N_cap = k_cache.shape[1], k_cache.shape[2]
    _need(k_cache, "k_cache", torch.bfloat16, (B, H_kv, N_cap, d), q.device)
    _need(v_cache, "v_cache", torch.bfloat16, (B, H_kv, N_cap, d), q.device)
    _need(kv_len, "kv_len", torch.int32, (B,), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, q.shape, q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H), q.device)
    _check(_lib.attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _ptr(kv_len), B, H,
                                    H_kv, N_cap, d, 0, float(scale), ATTN_BF16, _stream(q.device)))
    return out, lse


def decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                 kv_len: torch.Tensor, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 want_lse: bool = True):
    """Paged decode: q [B,H,d] bf16, pages [P,H_kv,page_size,d] bf16, block_table [B,max_pages] and
    kv_len [B] int32 on the GPU. Returns (o, lse)."""
    _need(q, "q", torch.bfloat16)
    B, H, d = q.shape
    P, H_kv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _need(k_pages, "k_pages", torch.bfloat16, (P, H_kv, page_size, d), q.device)
    _need(v_pages, "v_pages", torch.bfloat16, (P, H_kv, page_size, d), q.device)
    _need(block_table, "block_table", torch.int32, None, q.device)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    max_pages = block_table.shape[1]
    _need(kv_len, "kv_len", torch.int32, (B,), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, q.shape, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    need = decode_workspace_size(B, H, max_pages * page_size, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(_lib.attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(out), _ptr(lse), _ptr(kv_len),
                                  _ptr(block_table), B, H, H_kv, P, page_size, max_pages, d, float(scale), ATTN_BF16,
                                  _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out, lse


def bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.attn_bwd_workspace_size(B, H, N, d))


def bwd(q, k, v, o, dout, lse, causal: bool, scale: Optional[float] = None, dq=None, dk=None, dv=None,
        workspace: Optional[torch.Tensor] = None):
    """Backward: bf16 q, o, dout [B,H,N,d], k, v [B,H_kv,N,d] and fp32 lse [B,H,N] from fwd.

    Returns fp32 (dq [B,H,N,d], dk, dv [B,H_kv,N,d]); under grouped heads dk, dv sum over each KV
    head's query heads."""
    _need(q, "q", torch.bfloat16)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    for name, t in (("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, (B, H_kv, N, d), q.device)
    for name, t in (("o", o), ("dout", dout)):
        _need(t, name, torch.bfloat16, q.shape, q.device)
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32) if dq is None else dq
    dk = torch.empty(k.shape, **f32) if dk is None else dk
    dv = torch.empty(v.shape, **f32) if dv is None else dv
    _need(dq, "dq", torch.float32, q.shape, q.device)
    _need(dk, "dk", torch.float32, k.shape, q.device)
    _need(dv, "dv", torch.float32, v.shape, q.device)
    need = bwd_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(_lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                         B, H, H_kv, N, d, int(bool(causal)), float(scale), ATTN_BF16, _ptr(workspace),
                         workspace.numel(), _stream(q.device)))
    return dq, dk, dv


def bwd_varlen_workspace_size(T: int, H: int, d: int) -> int:
    return int(_lib.attn_bwd_varlen_workspace_size(T, H, d))


def bwd_varlen(q, k, v, o, dout, lse, cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool,
               scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace: Optional[torch.Tensor] = None):
    """Ragged backward: bf16 q, o, dout [T,H,d], k, v [T,H_kv,d], fp32 lse [H,T] from fwd_varlen and
    cu_seqlens [B+1] int32 on the GPU.

    Returns fp32 (dq [T,H,d], dk, dv [T,H_kv,d])."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q, k, v must be 3-D [T, H, d]")
    T, H, d = q.shape
    H_kv = k.shape[1]
    for name, t in (("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, (T, H_kv, d), q.device)
    for name, t in (("o", o), ("dout", dout)):
        _need(t, name, torch.bfloat16, q.shape, q.device)
    _need(lse, "lse", torch.float32, (H, T), q.device)
    _need(cu_seqlens, "cu_seqlens", torch.int32, None, q.device)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with B + 1 >= 2 entries")
    B = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32) if dq is None else dq
    dk = torch.empty(k.shape, **f32) if dk is None else dk
    dv = torch.empty(v.shape, **f32) if dv is None else dv
    _need(dq, "dq", torch.float32, q.shape, q.device)
    _need(dk, "dk", torch.float32, k.shape, q.device)
    _need(dv, "dv", torch.float32, v.shape, q.device)
    need = bwd_varlen_workspace_size(T, H, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(_lib.attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(cu_seqlens), B, int(max_seqlen), T, H, H_kv, d, int(bool(causal)),
                                float(scale), ATTN_BF16, _ptr(workspace), workspace.numel(), _stream(q.device)))
    return dq, dk, dv


def fwd_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.attn_fwd_bwd_workspace_size(B, H, N, d))


def fwd_bwd(q, k, v, dout, causal: bool, scale: Optional[float] = None, o=None, lse=None, dq=None, dk=None,
            dv=None, workspace: Optional[torch.Tensor] = None):
    """Forward and backward in one launch: bf16 q, dout [B,H,N,d], k, v [B,H_kv,N,d].

    Returns (o bf16 [B,H,N,d], lse fp32 [B,H,N], dq fp32 [B,H,N,d], dk, dv fp32 [B,H_kv,N,d])."""
    _need(q, "q", torch.bfloat16)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    for name, t in (("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, (B, H_kv, N, d), q.device)
    _need(dout, "dout", torch.bfloat16, q.shape, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    f32 = dict(dtype=torch.float32, device=q.device)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    lse = torch.empty((B, H, N), **f32) if lse is None else lse
    dq = torch.empty(q.shape, **f32) if dq is None else dq
    dk = torch.empty(k.shape, **f32) if dk is None else dk
    dv = torch.empty(v.shape, **f32) if dv is None else dv
    _need(o, "o", torch.bfloat16, q.shape, q.device)
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    _need(dq, "dq", torch.float32, q.shape, q.device)
    _need(dk, "dk", torch.float32, k.shape, q.device)
    _need(dv, "dv", torch.float32, v.shape, q.device)
    need = fwd_bwd_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(_lib.attn_fwd_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(o), _ptr(lse), _ptr(dq), _ptr(dk),
                             _ptr(dv), B, H, H_kv, N, d, int(bool(causal)), float(scale), ATTN_BF16,
                             _ptr(workspace), workspace.numel(), _stream(q.device)))
    return o, lse, dq, dk, dv


def timing_enable(on: bool = True) -> None:
    _check(_lib.attn_timing_enable(int(bool(on))))


def timing_reset() -> None:
    _check(_lib.attn_timing_reset())


def timing_read() -> dict:
    """{kernel name: (launches, total milliseconds)} for kernels timed since the last reset."""
    out = {}
    for i in range(_lib.attn_timing_count()):
        name = ctypes.c_char_p()
        n = ctypes.c_longlong()
        ms = ctypes.c_double()
        _check(_lib.attn_timing_get(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)))
        out[name.value.decode()] = (n.value, ms.value)
    return out


def timing_samples() -> dict:
    """{kernel name: [duration in ms of each launch, in launch order]} since the last reset."""
    out = {}
    for i in range(_lib.attn_timing_count()):
        name = ctypes.c_char_p()
        _check(_lib.attn_timing_get(i, ctypes.byref(name), None, None))
        n = _lib.attn_timing_samples(i, None, 0)
        if n < 0:
            raise AttnError(_lib.attn_last_error().decode())
        buf = (ctypes.c_float * max(n, 1))()
        got = _lib.attn_timing_samples(i, buf, n)
        if got < 0:
            raise AttnError(_lib.attn_last_error().decode())
        out[name.value.decode()] = [float(buf[j]) for j in range(min(got, n))]
    return out


def raw():
    """The loaded ctypes library (for ABI-level tests)."""
    return _lib
