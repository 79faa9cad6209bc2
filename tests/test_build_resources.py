"""Register use of the built kernels: no kernel of libmoe may spill to scratch.

The build reads hipcc's kernel-resource-usage remarks for every HIP source
(mixture_experts_layer_29_amd/build.py) and fails on any nonzero scratch size;
these tests check the remark parser and the report of the current build."""
import json
import os

import pytest

from mixture_experts_layer_29_amd import build as moe_build

REMARKS = """\
gemm_bf16.hip:501:1: remark: Function Name: _Z4kernAv [-Rpass-analysis=kernel-resource-usage]
gemm_bf16.hip:501:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
gemm_bf16.hip:501:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
gemm_bf16.hip:501:1: remark:     ScratchSize [bytes/lane]: 88 [-Rpass-analysis=kernel-resource-usage]
gemm_bf16.hip:501:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
gemm_bf16.hip:501:1: remark:     LDS Size [bytes/block]: 163840 [-Rpass-analysis=kernel-resource-usage]
route.hip:73:1: remark: Function Name: _Z4kernBv [-Rpass-analysis=kernel-resource-usage]
route.hip:73:1: remark:     VGPRs: 40 [-Rpass-analysis=kernel-resource-usage]
route.hip:73:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
route.hip:73:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
route.hip:73:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]
route.hip:73:1: remark:     LDS Size [bytes/block]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_remark_parser():
    u = moe_build.parse_resource_usage(REMARKS)
    assert u == {
        "_Z4kernAv": {"vgprs": 256, "agprs": 0, "scratch_bytes": 88, "waves_per_simd": 2,
                      "lds_bytes": 163840},
        "_Z4kernBv": {"vgprs": 40, "agprs": 0, "scratch_bytes": 0, "waves_per_simd": 8,
                      "lds_bytes": 0},
    }


def test_built_kernels_use_no_scratch():
    if not os.path.exists(moe_build.REPORT):
        pytest.skip("libmoe has not been built here (the build itself refuses spills)")
    with open(moe_build.REPORT) as f:
        usage = json.load(f)
    gemm = [k for k in usage if "moe_gemm_bf16" in k]
    assert gemm, "no grouped-GEMM kernel in the resource report"
    for name, u in usage.items():
        assert set(u) == {"vgprs", "agprs", "scratch_bytes", "waves_per_simd", "lds_bytes"}, name
        assert u["scratch_bytes"] == 0, f"{name} spills {u['scratch_bytes']} bytes per lane"
        assert u["vgprs"] + u["agprs"] <= 512, name
