"""The build refuses kernels that spill registers to scratch memory (spill
code in the 256-row expert-MLP kernels produced wrong results on gfx950), and
records hipcc's per-kernel resource report; these CPU tests check the report
parser and, when a build exists, the recorded report."""
import os

import pytest

from combine_group_limited_amd import build as B

SAMPLE = """\
x.hip:13:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]
x.hip:13:1: remark:     TotalSGPRs: 25 [-Rpass-analysis=kernel-resource-usage]
x.hip:13:1: remark:     VGPRs: 17 [-Rpass-analysis=kernel-resource-usage]
x.hip:13:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:13:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:13:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark: Function Name: _Z1jv [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     AGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     ScratchSize [bytes/lane]: 68 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     VGPRs Spill: 16 [-Rpass-analysis=kernel-resource-usage]
"""


def test_resource_report_parser():
    ks = B.kernel_resources(SAMPLE)
    assert [k["name"] for k in ks] == ["_Z1kv", "_Z1jv"]
    assert ks[0]["VGPRs"] == 17 and ks[0]["ScratchSize [bytes/lane]"] == 0
    assert ks[1]["AGPRs"] == 256 and ks[1]["ScratchSize [bytes/lane]"] == 68 and ks[1]["VGPRs Spill"] == 16


def test_built_kernels_use_no_scratch():
    if not os.path.exists(B.RESOURCES):
        pytest.skip("no build in this tree")
    lines = open(B.RESOURCES).read().splitlines()
    assert any("mlp_kernel" in l for l in lines) and any("combine" in l for l in lines)
    bad = [l for l in lines if "scratch=0 " not in l or not l.endswith("vgpr_spill=0")]
    assert not bad, bad
