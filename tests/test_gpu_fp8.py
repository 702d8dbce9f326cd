"""Parity of the fp8 (E4M3) forward with the fp64 oracle, through the C ABI.

The oracle computes exact attention of the real inputs (descale * decoded code). The tolerance is
derived, per output element, from the places where the kernel's arithmetic is not exact:

1. The probabilities that multiply V are rounded to E4M3, and the normaliser is the sum of those
   rounded values. Let M be the row's largest scaled score, p_j = exp(s_j - M) <= 1,
   l = sum_j p_j, w_j = p_j / l and O_c = sum_j w_j v_jc. On chip P_j = p_j * 2^(M - m + 6) with
   m <= M the running reference; rounding to nearest gives |P~_j - P_j| <= 2^-4 P_j for normal
   values (three mantissa bits) and <= 2^-10 for subnormal ones (spacing 2^-9). In units of p:
   |e_j| <= u p_j + a, u = 2^-4, a = 2^-16. As sum_j p_j (v_jc - O_c) = 0, the kernel's ratio
   sum_j p~_j v_jc / sum_j p~_j differs from O_c by sum_j e_j (v_jc - O_c) / sum_j p~_j, so
   |error| <= [u sum_j p_j |v_jc - O_c| + a sum_j |v_jc - O_c|] / (l (1 - u) - n a) for n valid keys.

2. The gfx950 E4M3 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4) does not sum its 64
   products exactly: measured on the device, products are summed in groups of 8 consecutive k
   slots, and within a group each product is truncated toward zero to 14 bits below the largest
   product of the group (so it loses less than 2^-13 of that maximum); groups and the
   accumulator add without that loss. One instruction therefore errs by at most
   t * sum_k |a_k b_k|, t = 2^-10. For P V that adds t (1 + u) / (1 - u) * sum_j w_j |v_jc|, for the
   normaliser (the same instruction against ones) a relative t, i.e. t |O_c|. For the scores it
   gives |ds_j| <= delta = t * |scale| * max_j sum_d |q_d k_jd| per row, which moves each softmax
   weight by a factor within exp(+-2 delta) and the LSE by at most delta.

  Worst case per element (sw = sum_j w_j |v_jc|, n valid keys, S1 = sum_j |v_jc|):
    |O~_c - O_c| <= e^(2 delta) [u (sw + |O_c|) + a (S1 + n |O_c|) / l] / (1 - u - n a / l)
                    + e^(2 delta) t (1 + u) / (1 - u) sw + t |O_c| + (e^(2 delta) - 1) (sw + |O_c|)
                    + 2^-9 |O_c| (bf16 output) + 1e-5 sw (float32 accumulation).
  |dLSE| <= delta + u + n a / l + t + 2e-5 per row (the log of the rounded normaliser's ratio).
  Every element must meet them. They assume every rounding at its extreme with one sign, so
  second checks bound the root mean squares: independent, zero-mean E4M3 roundings give
  E[err_c^2] <= sum_j (u p_j + a)^2 (v_jc - O_c)^2 / l^2 and E[dLSE^2] <= sum_j (u p_j + a)^2 / l^2;
  the score truncations enter as a variance too (at most 8 per group, each below 2^-13 of the group
  maximum), and the squared worst cases of the matrix-unit truncation and the bf16 output rounding
  are added. The measured RMS over all checked elements (and rows, for the LSE) must stay below the
  root mean of that expectation; this is the check that sees small systematic slips (a skipped
  tile moves every output a little).
"""

import numpy as np
import pytest
import torch

from oracle import attention as orc
from roofline_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

U8 = 2.0 ** -4    # E4M3 relative rounding bound (round to nearest, 3 mantissa bits)
A8 = 2.0 ** -16   # absolute rounding bound of subnormal P, relative to the row maximum
T8 = 2.0 ** -10   # per-instruction truncation of the E4M3 matrix unit, relative to sum |a_k b_k|


def real(t, descale):
    return float(descale) * orc.e4m3_decode(t.numpy())


def row_bounds(q, k, v, causal, scale, b, h, i_rows):
    """Bounds for rows i_rows of (b, h): (worst-case |dO| [n, d], expected |dO|^2 [n, d],
    worst-case |dLSE| [n], expected |dLSE|^2 [n])."""
    g = q.shape[1] // k.shape[1]
    kh, vh = k[b, h // g], v[b, h // g]
    i_rows = np.asarray(i_rows)
    s = scale * (q[b, h, i_rows] @ kh.T)  # [n, N]
    sabs = abs(scale) * (np.abs(q[b, h, i_rows]) @ np.abs(kh).T)
    if causal:
        keep = np.arange(kh.shape[0])[None, :] <= i_rows[:, None]
        s = np.where(keep, s, -np.inf)
        sabs = np.where(keep, sabs, 0.0)
    delta = T8 * sabs.max(axis=1, keepdims=True)
    e2 = np.exp(2 * delta)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    valid = np.isfinite(s).astype(np.float64)
    n = valid.sum(axis=1, keepdims=True)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ vh) / l
    ao = np.abs(o)
    av = np.abs(vh)
    sw = (p @ av) / l
    s1 = valid @ av
    den = 1 - U8 - A8 * n / l
    worst = (e2 * (U8 * (sw + ao) + A8 * (s1 + n * ao) / l) / den + e2 * T8 * (1 + U8) / (1 - U8) * sw + T8 * ao
             + (e2 - 1) * (sw + ao) + 2.0 ** -9 * ao + 1e-5 * sw)
    # variance model: E4M3 roundings against (v_j - O), score truncations (at most 8 per group, each
    # below 2^-13 of the group maximum, so E[ds^2] <= 2^-23 * scale^2 * sum_d (q_d k_d)^2; a weight
    # then moves by w_j (ds_j - sum_i w_i ds_i)), plus the squared worst cases of the truncation of
    # P V and of the normaliser and of the bf16 output rounding.
    sq = scale ** 2 * ((q[b, h, i_rows] ** 2) @ (kh ** 2).T)
    es2 = 2.0 ** -23 * np.where(np.isfinite(s), sq, 0.0).max(axis=1, keepdims=True)
    w2 = (p / l) ** 2
    var_s = es2 * (w2 @ vh ** 2 + 2 * ao * (w2 @ av) + ao ** 2 * w2.sum(axis=1, keepdims=True))
    r2 = (U8 * p + A8 * valid) ** 2
    dev2 = r2 @ (vh ** 2) - 2 * o * (r2 @ vh) + o ** 2 * r2.sum(axis=1, keepdims=True)  # sum r2 (v - O)^2
    var = dev2 / l ** 2 + var_s + (T8 * sw) ** 2 + (T8 * o) ** 2 + (2.0 ** -9 * o) ** 2
    lse_worst = delta[:, 0] + U8 + A8 * n[:, 0] / l[:, 0] + T8 + 2e-5
    lse_var = r2.sum(axis=1) / l[:, 0] ** 2 + es2[:, 0] * w2.sum(axis=1) + T8 ** 2 + 2e-5 ** 2
    return worst, var, lse_worst, lse_var


def check(o_gpu, lse_gpu, q, k, v, causal, scale, rows_by_head, ro, rl, label):
    """rows_by_head: list of (b, h, i_rows); ro/rl: oracle values in the same order."""
    og = I.to_f64(o_gpu)
    errs, worsts, vars_ = [], [], []
    gl, lse_tol, lse_vars = [], [], []
    for b, h, i_rows in rows_by_head:
        w, var, lt, lv = row_bounds(q, k, v, causal, scale, b, h, i_rows)
        errs.append(og[b, h, i_rows])
        worsts.append(w)
        vars_.append(var)
        lse_tol.append(lt)
        lse_vars.append(lv)
        gl.append(I.to_f64(lse_gpu)[b, h, i_rows])
    og_rows = np.concatenate(errs)
    err = np.abs(og_rows - ro)
    worst = np.concatenate(worsts)
    rms, rms_bound = float(np.sqrt(np.mean(err ** 2))), float(np.sqrt(np.mean(np.concatenate(vars_))))
    dl = np.abs(np.concatenate(gl) - rl)
    lt = np.concatenate(lse_tol)
    lrms, lrms_bound = float(np.sqrt(np.mean(dl ** 2))), float(np.sqrt(np.mean(np.concatenate(lse_vars))))
    el = float(np.max(dl))
    ratio = float(np.max(err / worst))
    print(f"{label}: max|dO|={err.max():.3e} max(err/bound)={ratio:.3f} rms={rms:.3e} "
          f"(model {rms_bound:.3e}) max|dLSE|={el:.3e} (bound {lt.min():.1e}..{lt.max():.1e}) "
          f"rms dLSE={lrms:.3e} (model {lrms_bound:.3e})")
    assert np.all(err <= worst), f"{label}: worst-case bound exceeded ({ratio:.3f})"
    assert rms <= rms_bound, f"{label}: rms error {rms:.3e} above the rounding model {rms_bound:.3e}"
    assert np.all(dl <= lt), f"{label}: LSE bound exceeded"
    assert lrms <= lrms_bound, f"{label}: LSE rms {lrms:.3e} above the rounding model {lrms_bound:.3e}"


def run(lib, t, causal, scale, descale=None):
    descale = t["descale"] if descale is None else descale
    o, lse = lib.fwd_fp8(t["q"].cuda(), t["k"].cuda(), t["v"].cuda(), descale, causal, scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def full_check(lib, t, causal, scale, descale, label):
    o, lse = run(lib, t, causal, scale, descale)
    q, k, v = (real(t[n], s) for n, s in zip("qkv", descale))
    ro, rl = orc.attention_fwd_fp8(t["q"].numpy(), t["k"].numpy(), t["v"].numpy(), descale, causal, scale)
    B, H, N, _ = q.shape
    rows = [(b, h, np.arange(N)) for b in range(B) for h in range(H)]
    check(o, lse, q, k, v, causal, scale, rows, ro.reshape(-1, q.shape[3]), rl.reshape(-1), label)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,H_kv,N,d", [(1, 2, 2, 333, 128), (2, 8, 2, 200, 128), (1, 2, 2, 1, 128),
                                           (1, 1, 1, 129, 128), (1, 2, 2, 600, 128), (2, 4, 4, 64, 128),
                                           (1, 4, 1, 127, 128), (1, 2, 2, 333, 64), (2, 4, 2, 200, 64),
                                           (1, 1, 1, 1, 64), (1, 2, 1, 600, 64)])
def test_fp8_shapes(lib, B, H, H_kv, N, d, causal):
    w = I.Workload("fp8_case", "fwd", B, H, H_kv, N, d, "e4m3", causal, seed=21)
    t = I.make_fp8_prefill(w)
    full_check(lib, t, causal, w.scale, t["descale"], f"fp8 B{B} H{H}/{H_kv} N{N} d{d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_arbitrary_descales_and_negative_scale(lib, causal):
    w = I.Workload("fp8_ds", "fwd", 1, 2, 1, 300, 128, "e4m3", causal, seed=22)
    t = I.make_fp8_prefill(w)
    ds = (t["descale"][0] * 1.37, -t["descale"][1] * 0.81, t["descale"][2] * 0.59)
    full_check(lib, t, causal, -0.07, ds, f"fp8 descales {ds} scale -0.07")


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_zero_scale_is_the_mean(lib, d):
    """scale 0: every probability is 2^6 exactly, so O is the mean of V up to the matrix unit's
    truncation (t * sum_j |v_j| / count) and the bf16 output rounding; LSE = ln(count)."""
    w = I.Workload("fp8_zero", "fwd", 1, 2, 2, 300, d, "e4m3", True, seed=23)
    t = I.make_fp8_prefill(w)
    o, lse = run(lib, t, True, 0.0)
    v = real(t["v"], t["descale"][2])
    count = np.arange(1, 301)[None, None, :, None]
    mean = np.cumsum(v, axis=2) / count
    trunc = T8 * np.cumsum(np.abs(v), axis=2) / count
    og = I.to_f64(o)
    err = np.abs(og - mean)
    print(f"zero scale: max|dO|={err.max():.3e} max rel={np.max(err / np.maximum(np.abs(mean), 1e-30)):.3e} "
          f"at {np.unravel_index(np.argmax(err - 2.0 ** -8 * np.abs(mean)), err.shape)} "
          f"max|mean|={np.abs(mean).max():.3e}")
    assert np.all(err <= trunc + 2.0 ** -8 * np.abs(mean) + 1e-7)
    np.testing.assert_allclose(I.to_f64(lse), np.log(np.arange(1, 301))[None, None, :].repeat(2, 1), atol=1e-5)


def test_fp8_causal_row0_and_one_hot_are_exact(lib):
    w = I.Workload("fp8_row0", "fwd", 1, 2, 2, 256, 128, "e4m3", True, seed=24)
    t = I.make_fp8_prefill(w)
    o, _ = run(lib, t, True, w.scale)
    v0 = torch.from_numpy(real(t["v"], t["descale"][2])[:, :, 0]).to(torch.bfloat16)  # E4M3 * 2^k fits bf16
    assert torch.equal(o[:, :, 0], v0)
    # one-hot: key j = unit vector e_(j mod 128) (code 0x38 = 1.0), query i = 16 * e_(i mod 128)
    # (code 0x58), scale 4: the selected score is 64, every other is 0, so P = (2^6, 0, ...).
    N, d = 128, 128
    k = torch.zeros(1, 1, N, d, dtype=torch.uint8)
    k[0, 0, torch.arange(N), torch.arange(N) % d] = 0x38
    q = torch.zeros(1, 1, N, d, dtype=torch.uint8)
    sel = (torch.arange(N) + 5) % d
    q[0, 0, torch.arange(N), sel] = 0x58
    v = t["v"][:1, :1, :N]
    one = {"q": q, "k": k, "v": v.contiguous(), "descale": (1.0, 1.0, t["descale"][2])}
    o1, _ = run(lib, one, False, 4.0)
    vr = torch.from_numpy(real(one["v"], t["descale"][2])).to(torch.bfloat16)
    assert torch.equal(o1[0, 0], vr[0, 0, sel])  # query i selects key (i + 5) mod 128 alone


def sample_rows(B, H, N, n_rand, seed):
    rng = np.random.default_rng(seed)
    fixed = [(0, 0, 0), (0, 0, 1), (B - 1, H - 1, N - 1), (0, H - 1, 127), (0, H - 1, 128), (B - 1, 0, 63),
             (B - 1, 0, 64), (0, 1, N // 2), (B - 1, H // 2, N - 129)]
    rnd = np.stack([rng.integers(0, B, n_rand), rng.integers(0, H, n_rand), rng.integers(0, N, n_rand)], 1)
    return np.concatenate([np.array(fixed), rnd])


@pytest.mark.parametrize("name", ["prefill_4k_causal_fp8", "prefill_4k_fp8"])
def test_fp8_prefill_4k_sampled_rows_and_a_head(lib, name):
    """The benchmarked workloads, in the benchmarked launch: 300+ sampled rows and all of head (1, 31)."""
    w = I.WORKLOADS[name]
    t = I.make_fp8_prefill(w)
    o, lse = run(lib, t, w.causal, w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    ds = t["descale"]
    q, k, v = (real(t[n], s) for n, s in zip("qkv", ds))
    groups = {}
    for b, h, i in sample_rows(w.B, w.H, w.N, 300, seed=7):
        groups.setdefault((int(b), int(h)), set()).add(int(i))
    groups.setdefault((1, 31), set()).update(range(w.N))
    rows_by_head = [(b, h, np.array(sorted(ii))) for (b, h), ii in sorted(groups.items())]
    flat = np.concatenate([np.stack([np.full(len(ii), b), np.full(len(ii), h), ii], 1) for b, h, ii in rows_by_head])
    ro, rl = orc.attention_fwd_fp8_rows(t["q"].numpy(), t["k"].numpy(), t["v"].numpy(), ds, w.causal, w.scale, flat)
    check(o, lse, q, k, v, w.causal, w.scale, rows_by_head, ro, rl, name)


def test_fp8_prefill_16k_sampled_rows(lib):
    """A long fp8 sequence (128 query tiles): sampled rows within the derived bound."""
    w = I.Workload("fp8_16k", "fwd", 1, 2, 2, 16384, 128, "e4m3", False, seed=28, qk_factor=0.5)
    t = I.make_fp8_prefill(w)
    o, lse = run(lib, t, w.causal, w.scale)
    ds = t["descale"]
    q, k, v = (real(t[n], s) for n, s in zip("qkv", ds))
    groups = {}
    for b, h, i in sample_rows(w.B, w.H, w.N, 100, seed=28):
        groups.setdefault((int(b), int(h)), set()).add(int(i))
    rows_by_head = [(b, h, np.array(sorted(ii))) for (b, h), ii in sorted(groups.items())]
    flat = np.concatenate([np.stack([np.full(len(ii), b), np.full(len(ii), h), ii], 1) for b, h, ii in rows_by_head])
    ro, rl = orc.attention_fwd_fp8_rows(t["q"].numpy(), t["k"].numpy(), t["v"].numpy(), ds, w.causal, w.scale, flat)
    check(o, lse, q, k, v, w.causal, w.scale, rows_by_head, ro, rl, "fp8_16k")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_rising_scores_take_both_softmax_paths(lib, causal):
    """Scores that rise from one 64-key tile to the next by 1.4 to 2.9 (log2 units): a rise of at
    most 2.86 leaves every probability finite in E4M3 (up to 2^8.86) on the path without the row
    maximum, a larger one overflows E4M3, turns a column sum NaN and takes the exact step. Every
    element stays within the derived bound, and the output is finite."""
    w = I.Workload("fp8_rise", "fwd", 1, 2, 2, 512, 128, "e4m3", causal, seed=25)
    t = I.make_fp8_prefill(w)
    # key tile j carries the exact E4M3 value ramp[j] in dimension 0, every query 1.0 there; scale 1
    ramp_codes = [0x00, 0x3C, 0x44, 0x48, 0x4C, 0x50, 0x52, 0x54]
    ramp_vals = [0.0, 1.5, 3.0, 4.0, 6.0, 8.0, 10.0, 12.0]
    assert np.array_equal(orc.e4m3_decode(np.array(ramp_codes, dtype=np.uint8)), np.array(ramp_vals))
    rises = np.diff(np.array(ramp_vals)) * 1.4426950408889634
    assert (rises <= 2.86).any() and (rises > 2.86).any() and (rises > 2.0).sum() >= 3
    # noise: dimensions 1..8 of every key hold random E4M3 values in [-1/2, 1/2] (every such code),
    # so scores within a tile are spread and their roundings behave as independent
    small = np.array([c for c in range(256) if c != 0x80 and abs(orc.e4m3_decode(np.array([c], dtype=np.uint8))[0]) <= 0.5
                      and np.isfinite(orc.e4m3_decode(np.array([c], dtype=np.uint8))[0])], dtype=np.uint8)
    rng = np.random.default_rng(5)
    q = torch.zeros_like(t["q"])
    q[..., 0:9] = 0x38
    k = torch.zeros_like(t["k"])
    for j in range(8):
        k[:, :, 64 * j:64 * j + 64, 0] = ramp_codes[j]
    k[..., 1:9] = torch.from_numpy(rng.choice(small, size=tuple(k.shape[:3]) + (8,)))
    case = {"q": q, "k": k, "v": t["v"], "descale": (1.0, 1.0, t["descale"][2])}
    # The reference the kernel keeps per row: the first tile's maximum, raised (by more than 2) to a
    # tile's maximum only when some 2^(s c - m + 6) of that tile does not fit E4M3 (above 464). All
    # queries here score every key alike, so outside the diagonal tile a wave's rows decide alike and
    # the per-row count below is the kernel's. Both outcomes occur.
    sc = (orc.e4m3_decode(q.numpy()) @ np.swapaxes(orc.e4m3_decode(k.numpy()), -1, -2)) * 1.4426950408889634
    fast_above_2 = exact_raise = 0
    for row in sc.reshape(-1, w.N, w.N):
        for i, srow in enumerate(row):
            n_keys = i + 1 if causal else w.N
            tiles = [srow[j:min(j + 64, n_keys)].max() for j in range(0, n_keys, 64)]
            m = tiles[0]
            for tm in tiles[1:]:
                if tm - m > np.log2(464.0) - 6:
                    exact_raise += 1
                    m = tm if tm > m + 2 else m
                elif tm - m > 2:
                    fast_above_2 += 1
    assert fast_above_2 > 0 and exact_raise > 0, (fast_above_2, exact_raise)
    o, lse = run(lib, case, causal, 1.0)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    full_check(lib, case, causal, 1.0, case["descale"], f"fp8 rising scores causal={causal}")
