"""The ceiling microbenchmarks run and land in physically sensible ranges (MI355X published
figures: dense bf16 2516.6 TFLOP/s, dense fp8 5033.2 TFLOP/s at 2.4 GHz, HBM3E 8 TB/s)."""
import pytest

from roofline_attention_amd import ceilings

pytestmark = pytest.mark.gpu


def test_ceilings_are_sensible():
    c = ceilings.measure()
    print(c)
    assert 0.3 * 2516.6 < c["mfma_bf16_tflops"] < 1.05 * 2516.6
    assert 0.3 * 5033.2 < c["mfma_fp8_tflops"] < 1.05 * 5033.2
    assert 20 < c["mfma_bf16_cycles_per_inst"] < 64 and 40 < c["mfma_fp8_cycles_per_inst"] < 128
    assert 0.4 * 8000 < c["hbm_read_gbs"] < 8000 and 0.3 * 8000 < c["hbm_copy_gbs"] < 8000
    assert 32 < c["lds_b128_bytes_per_clk_cu"] <= 256 and 32 < c["lds_tr_b16_bytes_per_clk_cu"] <= 256
    assert c["valu_exp_cycles"] >= c["valu_fma_cycles"] > 0
    # operands that switch like real data cannot run faster than near-constant ones, nor take a
    # different number of matrix-pipe cycles per instruction
    assert 0.3 * 2516.6 < c["mfma_bf16_random_tflops"] <= 1.02 * c["mfma_bf16_tflops"]
    assert 0.3 * 5033.2 < c["mfma_fp8_random_tflops"] <= 1.02 * c["mfma_fp8_tflops"]
    assert abs(c["mfma_bf16_random_cycles_per_inst"] - c["mfma_bf16_cycles_per_inst"]) < 2
    assert abs(c["mfma_fp8_random_cycles_per_inst"] - c["mfma_fp8_cycles_per_inst"]) < 4
    # the interleaved form can only be as fast as the slower of its two halves or slower
    assert c["coexec_cycles_interleaved"] >= 0.9 * max(c["coexec_cycles_mfma_only"], c["coexec_cycles_valu_only"])
