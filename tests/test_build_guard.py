"""The build refuses kernels that use scratch memory (register arrays that
fell out of registers); this checks the parsing of the compiler's
resource-usage remarks on sample text."""
from vision_mamba_selective_amd.build import scratch_kernels

LOG = """x.hip:1:1: remark: Function Name: kernel_a [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs: 80 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark: Function Name: kernel_b [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 768 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_kernels_found():
    assert scratch_kernels(LOG) == [("kernel_b", 768)]


def test_no_scratch():
    assert scratch_kernels(LOG.replace("768", "0")) == []
