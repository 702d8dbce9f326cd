"""Parity of the one-launch forward+backward (attn_fwd_bwd) with the fp64 oracle, through the C ABI.

The oracle is the one-pass forward+backward (attention_bwd returns dQ, dK, dV, O and LSE).
Tolerance: max abs error <= 2e-2 per output, as for the separate bf16 forward and backward.
The fused launch runs the same per-workgroup code as the separate kernels, so its O and LSE must
equal theirs bit for bit. Its gradients differ from theirs only through D (the same products of
the stored O and dO, summed in another order): a float32 rounding-level change, which the bf16
rounding of dS (an MFMA operand) can turn into one bf16 step (2^-8 relative) of some dS
elements, so fused and separate gradients are compared to 1e-3 (gradients here are of order 1).
"""
import numpy as np
import pytest
import torch

from oracle import attention as orc
from roofline_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def f64(t):
    return I.to_f64(t)


def max_err(gpu, ref):
    return float(np.max(np.abs(f64(gpu) - ref))) if ref.size else 0.0


def fused_case(lib, w):
    t = I.make_prefill(w, with_dout=True)
    q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "do"))
    out = lib.fwd_bwd(q, k, v, do, w.causal, w.scale)
    torch.cuda.synchronize()
    return t, [x.cpu() for x in out]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,H_kv,N,d", [(1, 2, 2, 256, 128), (1, 2, 2, 200, 128), (2, 2, 2, 333, 64),
                                           (1, 1, 1, 1, 128), (1, 2, 2, 65, 64), (1, 4, 2, 600, 128),
                                           (2, 8, 2, 333, 64), (1, 4, 1, 200, 128), (1, 8, 1, 129, 64)])
def test_fused_shapes(lib, B, H, H_kv, N, d, causal):
    w = I.Workload("fused_case", "fwdbwd", B, H, H_kv, N, d, "bf16", causal, seed=25)
    t, (o, lse, dq, dk, dv) = fused_case(lib, w)
    rdq, rdk, rdv, ro, rl = orc.attention_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]), causal, w.scale)
    errs = [max_err(o, ro), max_err(lse, rl), max_err(dq, rdq), max_err(dk, rdk), max_err(dv, rdv)]
    print(f"fused B{B} H{H}/{H_kv} N{N} d{d} causal={causal}: O, LSE, dQ, dK, dV errors {errs}")
    assert max(errs) <= TOL_BF16, errs


@pytest.mark.parametrize("causal", [False, True])
def test_fused_matches_separate_kernels(lib, causal):
    w = I.Workload("fused_vs_sep", "fwdbwd", 2, 4, 2, 700, 128, "bf16", causal, seed=26)
    t = I.make_prefill(w, with_dout=True)
    q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "do"))
    o1, l1, dq1, dk1, dv1 = lib.fwd_bwd(q, k, v, do, causal, w.scale)
    o2, l2 = lib.fwd(q, k, v, causal, w.scale)
    dq2, dk2, dv2 = lib.bwd(q, k, v, o2, do, l2, causal, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in ((dq1, dq2), (dk1, dk2), (dv1, dv2)):
        assert float((a - b).abs().max()) <= 1e-3


def test_fused_4k_causal_sampled_heads(lib):
    """The benchmarked fused workload in its benchmarked launch, two heads checked in full."""
    w = I.WORKLOADS["fwdbwd_4k_causal"]
    t, (o, lse, dq, dk, dv) = fused_case(lib, w)
    worst = [0.0] * 5
    for b, h in ((0, 0), (1, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rdq, rdk, rdv, ro, rl = orc.attention_bwd(f64(t["q"][sl]), f64(t["k"][sl]), f64(t["v"][sl]),
                                                  f64(t["do"][sl]), w.causal, w.scale)
        errs = [max_err(o[sl], ro), max_err(lse[sl], rl), max_err(dq[sl], rdq), max_err(dk[sl], rdk),
                max_err(dv[sl], rdv)]
        worst = [max(a, e) for a, e in zip(worst, errs)]
    print(f"fused fwdbwd_4k_causal: O, LSE, dQ, dK, dV errors {worst}")
    assert max(worst) <= TOL_BF16, worst
    for x in (o.float(), lse, dq, dk, dv):
        assert torch.isfinite(x).all()


def test_fused_is_deterministic_and_reuses_its_workspace(lib):
    """Phase-2 items go to whichever workgroup asks first; results must not depend on it. A second,
    smaller call on the same workspace (whose item counter the first call left behind) must match a
    call on a fresh workspace."""
    w = I.Workload("fdet", "fwdbwd", 1, 4, 4, 512, 128, "bf16", True, seed=27)
    t = I.make_prefill(w, with_dout=True)
    q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "do"))
    ws = torch.empty(lib.fwd_bwd_workspace_size(1, 4, 512, 128), dtype=torch.uint8, device="cuda")
    a = lib.fwd_bwd(q, k, v, do, True, w.scale, workspace=ws)
    b = lib.fwd_bwd(q, k, v, do, True, w.scale, workspace=ws)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    qs, ks, vs, dos = (x[:, :2, :300].contiguous() for x in (q, k, v, do))
    c = lib.fwd_bwd(qs, ks, vs, dos, True, w.scale, workspace=ws)
    d = lib.fwd_bwd(qs, ks, vs, dos, True, w.scale)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(c, d))
