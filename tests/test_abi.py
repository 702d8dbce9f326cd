"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and its
argument validation rejects bad calls before any HIP work is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
LIB = os.path.join(ROOT, "roofline_attention_amd", "libroofattn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libroofattn.so not built")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from roofline_attention_amd import binding
    return binding.raw()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def test_binding_signatures_cover_the_header():
    from roofline_attention_amd import binding
    assert sorted(binding.SIGNATURES) == declared_functions()


def test_version_and_status_strings(lib):
    assert lib.attn_abi_version() == 7
    assert lib.attn_status_string(OK) == b"ATTN_OK"
    assert lib.attn_status_string(WORKSPACE) == b"ATTN_ERR_WORKSPACE"
    assert lib.attn_status_string(99) == b"ATTN_ERR_UNKNOWN"


# Fake, well-aligned, non-overlapping device addresses: validation rejects each call below before
# any HIP call, so the addresses are never dereferenced.
BASE = 1 << 40
GAP = 1 << 34


def addr(i):
    return ctypes.c_void_p(BASE + i * GAP)


def fwd(lib, B=1, H=2, H_kv=2, N=128, d=64, causal=0, scale=0.125, dtype=BF16, ptrs=None):
    p = ptrs or [addr(i) for i in range(5)]
    return lib.attn_fwd(p[0], p[1], p[2], p[3], p[4], B, H, H_kv, N, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,want", [
    (dict(d=96), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
    (dict(H=3, H_kv=2), INVALID), (dict(N=0), INVALID), (dict(B=0), INVALID), (dict(H_kv=0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID), (dict(N=1 << 24, d=128), INVALID),
])
def test_fwd_rejects_bad_arguments(lib, kw, want):
    assert fwd(lib, **kw) == want
    assert lib.attn_last_error() != b""


def test_fwd_rejects_null_misaligned_and_overlapping(lib):
    p = [addr(i) for i in range(5)]
    assert fwd(lib, ptrs=[None] + p[1:]) == INVALID
    mis = list(p)
    mis[1] = ctypes.c_void_p(BASE + GAP + 8)
    assert fwd(lib, ptrs=mis) == INVALID
    ov = list(p)
    ov[3] = ctypes.c_void_p(BASE + 64)  # output inside q
    assert fwd(lib, ptrs=ov) == INVALID
    ov = list(p)
    ov[4] = ctypes.c_void_p(BASE + 3 * GAP + 16)  # lse inside o
    assert fwd(lib, ptrs=ov) == INVALID


def fwd_fp8(lib, B=1, H=2, H_kv=2, N=128, d=128, causal=0, scale=0.125, ds=(1.0, 1.0, 1.0), ptrs=None):
    p = ptrs or [addr(i) for i in range(5)]
    return lib.attn_fwd_fp8(p[0], p[1], p[2], p[3], p[4], B, H, H_kv, N, d, causal, scale, *ds, None)


@pytest.mark.parametrize("kw,want", [
    (dict(d=32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(H=3, H_kv=2), INVALID), (dict(N=0), INVALID),
    (dict(ds=(float("nan"), 1.0, 1.0)), INVALID), (dict(ds=(1.0, float("inf"), 1.0)), INVALID),
    (dict(ds=(1.0, 1.0, float("-inf"))), INVALID), (dict(scale=1e30, ds=(1e30, 1e30, 1.0)), INVALID),
    (dict(scale=float("nan")), INVALID),
])
def test_fwd_fp8_rejects_bad_arguments(lib, kw, want):
    assert fwd_fp8(lib, **kw) == want
    assert lib.attn_last_error() != b""


def test_fwd_fp8_rejects_null_misaligned_and_overlapping(lib):
    p = [addr(i) for i in range(5)]
    assert fwd_fp8(lib, ptrs=[None] + p[1:]) == INVALID
    mis = list(p)
    mis[2] = ctypes.c_void_p(BASE + 2 * GAP + 4)
    assert fwd_fp8(lib, ptrs=mis) == INVALID
    # o (bf16, 2 bytes per element) overlapping the end of q's uint8 range
    ov = list(p)
    ov[3] = ctypes.c_void_p(BASE + 2 * 128 * 128 - 16)
    assert fwd_fp8(lib, ptrs=ov) == INVALID


def test_fwd_varlen_validation(lib):
    p = [addr(i) for i in range(6)]

    def call(B=3, max_seqlen=100, T=250, H=4, H_kv=2, d=128, dtype=BF16, cu=p[5], lse=p[4]):
        return lib.attn_fwd_varlen(p[0], p[1], p[2], p[3], lse, cu, B, max_seqlen, T, H, H_kv, d, 1, 0.088, dtype,
                                   None)

    assert call(cu=None) == INVALID
    assert call(T=-1) == INVALID
    assert call(B=0) == INVALID
    assert call(max_seqlen=0) == INVALID
    assert call(H=4, H_kv=3) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(dtype=F32) == UNSUPPORTED
    assert call(cu=ctypes.c_void_p(BASE + 5 * GAP + 2)) == INVALID  # misaligned offsets
    assert call(lse=ctypes.c_void_p(BASE + 3 * GAP + 64)) == INVALID  # lse inside o
    assert call(T=0) == OK  # no rows: nothing is launched


def test_bwd_varlen_validation(lib):
    p = [addr(i) for i in range(11)]
    T, H, d = 250, 4, 128
    need = lib.attn_bwd_varlen_workspace_size(T, H, d)
    assert need == 2 * H * T * 4  # D and LSE * log2 e per (head, token) row

    def call(B=3, max_seqlen=100, T=T, H=H, H_kv=2, d=d, dtype=BF16, cu=p[9], ws=p[10], ws_bytes=need, lse=p[5]):
        return lib.attn_bwd_varlen(p[0], p[1], p[2], p[3], p[4], lse, p[6], p[7], p[8], cu, B, max_seqlen, T, H,
                                   H_kv, d, 1, 0.088, dtype, ws, ws_bytes, None)

    assert call(cu=None) == INVALID
    assert call(lse=None) == INVALID
    assert call(T=-1) == INVALID
    assert call(B=0) == INVALID
    assert call(max_seqlen=0) == INVALID
    assert call(H=4, H_kv=3) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(dtype=F32) == UNSUPPORTED
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(cu=ctypes.c_void_p(BASE + 9 * GAP + 2)) == INVALID  # misaligned offsets
    assert call(ws=ctypes.c_void_p(BASE + 6 * GAP + 64)) == INVALID  # workspace inside dq
    assert call(lse=ctypes.c_void_p(BASE + 7 * GAP)) == INVALID  # lse (an input) is dk (an output)
    assert call(T=0, ws=None, ws_bytes=0) == OK  # no rows: nothing is launched


def test_decode_validation(lib):
    p = [addr(i) for i in range(7)]
    ws_need = lib.attn_decode_workspace_size(64, 32, 8192, 128)
    assert ws_need == 64 * 32 * 9 * (128 + 4) * 4  # ceil(8192 / 1024) + 1 record slots

    def call(B=64, H=32, H_kv=8, N_cap=8192, d=128, dtype=BF16, ws=p[6], ws_bytes=ws_need, kv=p[5]):
        return lib.attn_decode(p[0], p[1], p[2], p[3], p[4], kv, B, H, H_kv, N_cap, d, 0, 0.088, dtype, ws,
                               ws_bytes, None)

    assert call(ws_bytes=ws_need - 1) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(dtype=F32) == UNSUPPORTED
    assert call(B=65535, H=4352, H_kv=256) == INVALID  # groups of 17: two 16-head chunks, beyond one grid row
    assert call(H=30) == INVALID
    assert call(kv=None) == INVALID
    assert call(d=80) == UNSUPPORTED
    assert call(B=65535, H=512, H_kv=512) == INVALID  # B * H_kv beyond one grid row
    assert lib.attn_decode_workspace_size(1, 1, 1, 96) == 0


def test_decode_noalloc_validation(lib):
    # rejected before any HIP call: bad arguments as for attn_decode, and shapes whose split records
    # exceed the library's fixed 16 MiB scratch
    p = [addr(i) for i in range(6)]

    def call(B=64, H=32, H_kv=8, N_cap=8192, d=128, dtype=BF16, ptrs=None):
        q = ptrs if ptrs is not None else p
        return lib.attn_decode_noalloc(*q, B, H, H_kv, N_cap, d, 0, 0.088, dtype, None)

    assert call(N_cap=16384) == WORKSPACE  # 64 x 32 x 17 record slots x 528 B = 18.4 MB
    assert b"scratch" in lib.attn_last_error()
    assert call(d=96) == UNSUPPORTED
    assert call(dtype=F32) == UNSUPPORTED
    assert call(H=30) == INVALID
    assert call(ptrs=p[:5] + [None]) == INVALID  # kv_len is required
    ov = list(p)
    ov[3] = p[0]  # o on top of q
    assert call(ptrs=ov) == INVALID


def test_decode_paged_validation(lib):
    p = [addr(i) for i in range(8)]
    ws_need = lib.attn_decode_workspace_size(64, 32, 128 * 64, 128)

    def call(H=32, H_kv=8, P=1000, ps=64, max_pages=128, d=128, dtype=BF16, table=p[6], ws_bytes=ws_need):
        return lib.attn_decode_paged(p[0], p[1], p[2], p[3], p[4], p[5], table, 64, H, H_kv, P, ps, max_pages, d,
                                     0.088, dtype, p[7], ws_bytes, None)

    assert call(table=None) == INVALID
    assert call(ps=16) == UNSUPPORTED
    assert call(ps=96) == UNSUPPORTED
    assert call(ps=2048) == UNSUPPORTED
    assert call(P=0) == INVALID
    assert call(max_pages=0) == INVALID
    assert call(ws_bytes=ws_need - 4) == WORKSPACE
    assert call(dtype=F32) == UNSUPPORTED
    assert call(table=ctypes.c_void_p(BASE + 6 * GAP + 2)) == INVALID


def test_bwd_validation(lib):
    p = [addr(i) for i in range(11)]
    need = lib.attn_bwd_workspace_size(2, 16, 4096, 128)
    assert need == 2 * 2 * 16 * 4096 * 4  # D and LSE*log2(e) per query row

    def call(H=16, H_kv=16, dtype=BF16, ws_bytes=need, lse=p[5]):
        return lib.attn_bwd(p[0], p[1], p[2], p[3], p[4], lse, p[6], p[7], p[8], 2, H, H_kv, 4096, 128, 1, 0.088,
                            dtype, p[9], ws_bytes, None)

    assert call(ws_bytes=need - 4) == WORKSPACE
    assert call(H_kv=5) == INVALID  # 16 query heads do not split into 5 groups
    assert call(dtype=F32) == UNSUPPORTED
    assert call(lse=None) == INVALID


def test_fwd_bwd_validation(lib):
    p = [addr(i) for i in range(10)]
    ws_need = lib.attn_fwd_bwd_workspace_size(1, 2, 128, 64)
    assert ws_need == 2 * 2 * 128 * 4 + 16
    assert lib.attn_fwd_bwd_workspace_size(1, 2, 128, 96) == 0

    def call(B=1, H=2, H_kv=2, N=128, d=64, dtype=BF16, ws_bytes=ws_need, ptrs=p):
        return lib.attn_fwd_bwd(*ptrs[:9], B, H, H_kv, N, d, 1, 0.125, dtype, ptrs[9], ws_bytes, None)

    assert call(dtype=F32) == UNSUPPORTED
    assert call(d=96) == UNSUPPORTED
    assert call(H=3) == INVALID
    assert call(ws_bytes=ws_need - 1) == WORKSPACE
    assert call(ptrs=p[:5] + [None] + p[6:]) == INVALID  # lse is required
    ov = list(p)
    ov[6] = p[0]  # dq on top of q
    assert call(ptrs=ov) == INVALID


def test_timer_without_launches(lib):
    assert lib.attn_timing_reset() == OK
    assert lib.attn_timing_count() == 0
    assert lib.attn_timing_get(0, None, None, None) == INVALID
    assert lib.attn_timing_samples(0, None, 0) == -1
    assert lib.attn_timing_samples(-1, None, 0) == -1


def test_release_without_launches_is_a_no_op(lib):
    # no event was ever created: nothing to wait for or destroy, and no HIP call is made
    assert lib.attn_release() == OK
    assert lib.attn_release() == OK
    assert lib.attn_timing_count() == 0
