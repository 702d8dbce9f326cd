"""The analytic ledger against the values the pages print (tests/golden/ledger_pins.json)."""
import json
import math
import os

import pytest

from roofline_attention_amd import ledger as L

PINS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ledger_pins.json")))


def test_naive_intensity_limit_and_fraction():
    p = PINS["naive_intensity_limit"]
    lim = L.naive_intensity(10**9, p["d"], p["s"])
    assert lim == pytest.approx(p["value"], rel=1e-6)
    assert L.naive_intensity(4096, 128, 2) < lim  # the plateau is approached from below
    f = PINS["naive_fraction_of_h100"]
    assert round(lim / f["ridge"], 3) == f["value"]


def test_compulsory_tiled_decode_gqa():
    p = PINS["compulsory_intensity"]
    assert L.compulsory_intensity(p["N"], p["s"]) == p["value"]
    # the compulsory bytes of one head's forward give the same intensity: 4 N^2 d / (4 s N d)
    N, d = p["N"], 128
    assert L.fwd_flops(1, 1, N, d, False) / L.fwd_bytes(1, 1, 1, N, d, p["s"], lse=False) == p["value"]
    t = PINS["tiled_intensity_limit"]
    assert L.tiled_intensity(10**7, 128, t["s"], t["B_r"]) == pytest.approx(t["value"], rel=1e-4)
    dd = PINS["decode_intensity"]
    assert L.decode_intensity(dd["g"], dd["s"]) == dd["value"]
    assert L.decode_flops(1, 128, [1000]) / L.decode_bytes(1, 1, 128, 2, [1000], lse=False) == pytest.approx(1.0, rel=1e-2)
    gq = PINS["gqa_intensity"]
    assert L.decode_intensity(gq["g"], gq["s"]) == gq["value"]


def test_moa_naive_bytes():
    p = PINS["moa_naive_forward_bytes"]
    r, w, t = L.moa_naive_fwd_bytes(p["B"], p["N"], p["D"], p["s"])
    assert round(r / 1e6, 3) == p["read_mb"]
    assert round(w / 1e6, 3) == p["write_mb"]
    assert round(t / 1e6, 3) == p["total_mb"]


def test_fusion_round_trip():
    p = PINS["fusion_round_trip_bytes"]
    assert L.round_trip_bytes(p["M"], p["N"], p["s"]) == p["value"]


def test_causal_halving_and_backward_ratio():
    assert L.fwd_flops(2, 32, 4096, 128, True) * 2 == L.fwd_flops(2, 32, 4096, 128, False)
    assert L.bwd_flops(2, 16, 4096, 128, True) == 2.5 * L.fwd_flops(2, 16, 4096, 128, True)
    assert math.isclose(L.fwd_flops(2, 32, 4096, 128, True), 274.877906944e9)
