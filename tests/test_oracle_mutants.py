"""Planted mistakes in the oracle, on the CPU: each must fail at least one pin.

Each mutant is the oracle's own source with one plausible slip edited in (a
dropped term, a wrong sign or index, a transposed operand, an off-by-one mask).
The mutated copy is loaded as a separate module and the pin suite of
test_oracle_pins is run against it; a mutant that passes every pin would mean the
pins cannot tell that slip from the correct oracle.
"""
import importlib.util
import inspect
import os
import types

import pytest

import oracle.attention as real_oracle
from tests import test_oracle_pins as pins

SRC = inspect.getsource(real_oracle)

MUTANTS = {
    "mask_drops_diagonal": ("np.triu(np.ones((n_q, n_k), dtype=bool), k=1)", "np.triu(np.ones((n_q, n_k), dtype=bool), k=0)"),
    "mask_ignored": ("    if causal:\n        n_q, n_k = s.shape", "    if False:\n        n_q, n_k = s.shape"),
    "scale_dropped": ("s = scale * (qh @ kh.T)", "s = (qh @ kh.T)"),
    "operand_transposed": ("s = scale * (qh @ kh.T)", "s = scale * (kh @ qh.T)"),
    "softmax_wrong_axis": ("l = e.sum(axis=1, keepdims=True)", "l = e.sum(axis=0, keepdims=True)"),
    "lse_missing_max": ("lse = (m + np.log(l))[:, 0]", "lse = (np.log(l))[:, 0]"),
    "gqa_modulo_map": ("            hk = h // g\n            s = _scores", "            hk = h % H_kv\n            s = _scores"),
    "bwd_output_uses_unnormalised_p": ("            o[b, h] = p @ v[b, hk]\n            dv[b, hk] += p.T @ dout[b, h]",
                                       "            o[b, h] = np.exp(s - s.max(axis=1, keepdims=True)) @ v[b, hk]\n            dv[b, hk] += p.T @ dout[b, h]"),
    "bwd_drops_D": ("ds = p * (dp - D)", "ds = p * dp"),
    "bwd_sign": ("ds = p * (dp - D)", "ds = p * (D - dp)"),
    "bwd_dk_no_scale": ("dk[b, hk] += scale * (ds.T @ q[b, h])", "dk[b, hk] += (ds.T @ q[b, h])"),
    "bwd_dv_transposed": ("dv[b, hk] += p.T @ dout[b, h]", "dv[b, hk] += p @ dout[b, h]"),
    "rows_causal_off_by_one": ("n_keys = i + 1 if causal else N", "n_keys = i if causal else N"),
    "varlen_crosses_sequences": ("s = _scores(q[r0:r1, h], k[r0:r1, hk], causal, scale)",
                                 "s = _scores(q[r0:r1, h], k[:r1, hk], causal, scale)"),
    "varlen_rows_global_causal": ("k_end = t + 1 if causal else r1", "k_end = t + 1 - r0 if causal else r1"),
    "varlen_bwd_dk_overwrites_group": ("dk[r0:r1, hk] += scale * (ds.T @ qs)", "dk[r0:r1, hk] = scale * (ds.T @ qs)"),
    "varlen_bwd_drops_D": ("ds = p * (dp - np.sum(dos * os_, axis=1, keepdims=True))", "ds = p * dp"),
    "varlen_bwd_gqa_modulo_map": ("            hk = h // g\n            qs, ks", "            hk = h % H_kv\n            qs, ks"),
    "varlen_bwd_dv_not_transposed": ("dv[r0:r1, hk] += p.T @ dos", "dv[r0:r1, hk] += p @ dos"),
    "paged_wrong_page": ("pages = table[b, :(n + ps - 1) // ps]", "pages = table[b, 1:(n + ps - 1) // ps + 1]"),
    "paged_reads_first_head": ("np.asarray(k_pages[p, hk], dtype=np.float64) for p in pages",
                               "np.asarray(k_pages[p, 0], dtype=np.float64) for p in pages"),
    "e4m3_bias_8": ("(1.0 + m / 8.0) * np.exp2(e - 7.0)", "(1.0 + m / 8.0) * np.exp2(e - 8.0)"),
    "e4m3_subnormal_implicit_one": ("(m / 8.0) * 2.0 ** -6", "(1.0 + m / 8.0) * 2.0 ** -6"),
    "e4m3_sign_threshold_off_by_one": ("sign = np.where(c >= 128, -1.0, 1.0)", "sign = np.where(c >= 129, -1.0, 1.0)"),
    "fp8_v_descale_dropped": ("dq * e4m3_decode(q8), dk * e4m3_decode(k8), dv * e4m3_decode(v8)",
                              "dq * e4m3_decode(q8), dk * e4m3_decode(k8), e4m3_decode(v8)"),
    "fp8_k_uses_q_descale": ("dq * e4m3_decode(q8), dk * e4m3_decode(k8), dv * e4m3_decode(v8)",
                             "dq * e4m3_decode(q8), dq * e4m3_decode(k8), dv * e4m3_decode(v8)"),
    "decode_reads_one_short": ("kh = np.asarray(k_cache[b, hk, :n], dtype=np.float64)",
                               "kh = np.asarray(k_cache[b, hk, :n - 1], dtype=np.float64)"),
}

# The pin suite, with the parameters each pin runs at.
PIN_CALLS = [
    (pins.test_fwd_matches_torch_sdpa, dict(B=2, H=4, H_kv=2, N=37, d=16, causal=False)),
    (pins.test_fwd_matches_torch_sdpa, dict(B=2, H=4, H_kv=2, N=37, d=16, causal=True)),
    (pins.test_fwd_scale_zero_is_uniform_average, dict(causal=True)),
    (pins.test_fwd_single_key, {}),
    (pins.test_fwd_rows_sum_to_one, {}),
    (pins.test_fwd_constant_v, dict(causal=True)),
    (pins.test_fwd_causal_row0, {}),
    (pins.test_fwd_one_hot_selection_and_exact_lse, {}),
    (pins.test_fwd_key_shift_moves_lse_only, dict(causal=True)),
    (pins.test_fwd_gqa_equals_expanded_heads, {}),
    (pins.test_fwd_rows_agree_with_full, dict(causal=True)),
    (pins.test_decode_matches_sdpa_single_query_and_ignores_pad, {}),
    (pins.test_decode_is_last_causal_row, {}),
    (pins.test_bwd_matches_torch_autograd, dict(B=2, H=4, H_kv=2, N=23, d=8, causal=True)),
    (pins.test_bwd_sum_invariants, dict(causal=True)),
    (pins.test_bwd_returns_the_forward, dict(causal=True)),
    (pins.test_bwd_constant_v_and_zero_scale, {}),
    (pins.test_bwd_causal_last_key, {}),
    (pins.test_varlen_equals_block_diagonal_mask, dict(causal=True, H=4, H_kv=2)),
    (pins.test_varlen_rows_agree_with_full, dict(causal=True)),
    (pins.test_varlen_bwd_matches_autograd_with_block_diagonal_mask, dict(causal=True, H=4, H_kv=2)),
    (pins.test_varlen_bwd_finite_differences, {}),
    (pins.test_decode_paged_equals_contiguous, dict(shuffle=True)),
    (pins.test_decode_paged_matches_sdpa, {}),
    (pins.test_e4m3_decode_matches_torch_on_every_code, {}),
    (pins.test_e4m3_decode_closed_forms, {}),
    (pins.test_fp8_fwd_matches_torch_decode_and_sdpa, dict(causal=True)),
    (pins.test_fp8_descales_enter_as_exact_factors, {}),
    (pins.test_fp8_rows_agree_with_full, {}),
]


def load_mutant(name: str) -> types.ModuleType:
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def pins_fail(mod) -> list:
    failed = []
    saved = pins.orc
    pins.orc = mod
    try:
        for fn, kw in PIN_CALLS:
            try:
                fn(**kw)
            except Exception as e:  # an assertion, or a crash the slip causes
                failed.append((fn.__name__, type(e).__name__))
    finally:
        pins.orc = saved
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert pins_fail(real_oracle) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    failed = pins_fail(load_mutant(name))
    assert failed, f"mutant {name} passed every pin"
