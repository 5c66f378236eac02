"""The build's register-spill check: parsing of the compiler's kernel resource report."""

import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def builder():
    spec = importlib.util.spec_from_file_location("_temx_build_t", os.path.join(ROOT, "mxfp8_mixed_precision_amd",
                                                                                 "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


REPORT = """\
gemm.hip:10:1: remark: Function Name: _Z6kernelAv [-Rpass-analysis=kernel-resource-usage]
gemm.hip:10:1: remark:     VGPRs: 200 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:20:1: remark: Function Name: _Z6kernelBv [-Rpass-analysis=kernel-resource-usage]
gemm.hip:20:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
gemm.hip:20:1: remark:     ScratchSize [bytes/lane]: 68 [-Rpass-analysis=kernel-resource-usage]
warning: '-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)
gemm.hip:30:1: remark: Function Name: _Z6kernelCv [-Rpass-analysis=kernel-resource-usage]
gemm.hip:30:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
"""


def test_spilled_kernels_lists_exactly_the_kernels_with_scratch():
    assert builder().spilled_kernels(REPORT) == [("_Z6kernelBv", 68), ("_Z6kernelCv", 16)]


def test_spilled_kernels_empty_report():
    assert builder().spilled_kernels("") == []
