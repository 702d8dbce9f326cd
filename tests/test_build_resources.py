"""The compiled kernels' resources, from the compiler's per-kernel report that build() records.

No kernel of the library may spill vector registers to scratch memory, and the kernels whose
design rests on a number of waves per SIMD must keep it: the bf16 forward at d = 128 and the dQ
kernel at d = 128 two waves, the dK/dV kernel one wave at d = 128 (accumulators in AGPRs) and two
at d = 64, the d = 64 forward three.
"""
import json
import os

import pytest

from roofline_attention_amd import build as B

REMARKS = """\
x.hip:25:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
x.hip:25:1: remark:     TotalSGPRs: 32 [-Rpass-analysis=kernel-resource-usage]
x.hip:25:1: remark:     VGPRs: 202 [-Rpass-analysis=kernel-resource-usage]
x.hip:25:1: remark:     AGPRs: 16 [-Rpass-analysis=kernel-resource-usage]
x.hip:25:1: remark:     ScratchSize [bytes/lane]: 48 [-Rpass-analysis=kernel-resource-usage]
x.hip:25:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]
x.hip:25:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
x.hip:25:1: remark:     SGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
x.hip:25:1: remark:     VGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]
x.hip:25:1: remark:     LDS Size [bytes/block]: 32768 [-Rpass-analysis=kernel-resource-usage]
x.hip:40:1: remark: Function Name: _Z3barv [-Rpass-analysis=kernel-resource-usage]
x.hip:40:1: remark:     VGPRs: 8 [-Rpass-analysis=kernel-resource-usage]
x.hip:40:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_parse_resources():
    r = B.parse_resources(REMARKS)
    assert r == {
        "_Z3fooPf": {"vgprs": 202, "agprs": 16, "scratch_bytes_per_lane": 48, "waves_per_simd": 2,
                     "sgpr_spills": 3, "vgpr_spills": 12, "static_lds_bytes": 32768},
        "_Z3barv": {"vgprs": 8, "scratch_bytes_per_lane": 0},
    }


@pytest.fixture(scope="module")
def resources():
    path = B.resources_path()
    if not os.path.exists(path):
        pytest.skip("library not built (python -m roofline_attention_amd.build)")
    with open(path) as f:
        return json.load(f)


def _find(res, kernel, hd, *flags):
    """Resource entries of kernel `kernel` instantiated at head dimension hd with leading bool flags."""
    tag = f"{kernel}ILi{hd}E" + "".join(f"Lb{int(b)}E" for b in flags)
    found = {k: v for k, v in res.items() if tag in k}
    assert found, f"no kernel matching {tag}"
    return found


def test_every_kernel_reported(resources):
    for kernel in ("fwd_bf16_kernel", "fwd_fp8_kernel", "fwd_f32_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel",
                   "bwd_dq_varlen_kernel", "bwd_dkdv_varlen_kernel", "fwdbwd_kernel", "decode_split_kernel",
                   "decode_combine_kernel"):
        assert any(kernel in k for k in resources), kernel


def test_no_kernel_spills_to_scratch(resources):
    bad = {k: v for k, v in resources.items() if v.get("scratch_bytes_per_lane", 0) or v.get("vgpr_spills", 0)}
    assert not bad, bad


@pytest.mark.parametrize("kernel,hd,flags,waves", [
    ("fwd_bf16_kernel", 128, (), 2),
    ("fwd_bf16_kernel", 64, (), 3),
    ("bwd_dq_kernel", 128, (), 2),
    ("bwd_dkdv_kernel", 128, (), 1),
    ("bwd_dkdv_kernel", 64, (), 2),
])
def test_waves_per_simd(resources, kernel, hd, flags, waves):
    for name, v in _find(resources, kernel, hd, *flags).items():
        assert v["waves_per_simd"] >= waves, (name, v)
