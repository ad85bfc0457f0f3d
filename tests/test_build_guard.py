"""The build's scratch guard (block_sparse_attention_fmha_amd/build.py) reads hipcc's
resource-usage remarks: a kernel with scratch memory or spilled VGPRs is reported (and
stops the build); SGPR spills, which go to VGPR lanes, are not."""
from block_sparse_attention_fmha_amd.build import kernels_using_scratch

REMARKS = """x.hip:1:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark: Function Name: _Z3bazPf [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     SGPRs Spill: 6 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark: Function Name: _Z3barPf [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 52 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_kernels_are_reported():
    assert kernels_using_scratch(REMARKS) == [("_Z3barPf", "VGPRs Spill", 12),
                                              ("_Z3barPf", "ScratchSize [bytes/lane]", 52)]


def test_clean_remarks_pass():
    assert kernels_using_scratch(REMARKS.split("x.hip:9:1")[0]) == []
