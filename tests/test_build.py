"""Host-side checks of the build script: its scan of the compiler's
per-kernel resource report for scratch memory."""
from paged_kv_decode_pa_amd import build as B

REPORT = """\
x.h:10:1: remark: Function Name: _ZN2pa3fooEv [-Rpass-analysis=kernel-resource-usage]
x.h:10:1: remark:     VGPRs: 162 [-Rpass-analysis=kernel-resource-usage]
x.h:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.h:20:1: remark: Function Name: _ZN2pa3barEv [-Rpass-analysis=kernel-resource-usage]
x.h:20:1: remark:     ScratchSize [bytes/lane]: 272 [-Rpass-analysis=kernel-resource-usage]
x.h:30:1: remark: Function Name: _ZN2pa18decode_mfma_kernelILi2ELi256ELi8ELi1ELb1ELb1EEEvNS_12DecodeParamsE [-Rpass-analysis=kernel-resource-usage]
x.h:30:1: remark:     ScratchSize [bytes/lane]: 60 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_kernels_flags_new_scratch_only():
    assert B.scratch_kernels(REPORT) == [("_ZN2pa3barEv", 272)]


def test_scratch_kernels_empty_report():
    assert B.scratch_kernels("") == []
