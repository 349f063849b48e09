"""The compiler's per-kernel resource report: no kernel may use scratch
memory or spill registers (a scratch load waits behind every streamed cache
load in flight), and every decode kernel keeps at least two waves per SIMD."""
import os

import pytest

from quantized_kv_cache_06_amd import build as B

REMARKS = """x.hip:1:1: remark: Function Name: _Z4goodv [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs: 100 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     Occupancy [waves/SIMD]: 4 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark: Function Name: _Z3badv [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs: 160 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 48 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_report_parser_and_check():
    k = B.parse_resource_usage(REMARKS)
    assert set(k) == {"_Z4goodv", "_Z3badv"}
    assert k["_Z4goodv"]["Occupancy [waves/SIMD]"] == "4"
    assert k["_Z3badv"]["ScratchSize [bytes/lane]"] == "48"
    B.check_resource_usage({"_Z4goodv": k["_Z4goodv"]})
    with pytest.raises(RuntimeError, match="_Z3badv"):
        B.check_resource_usage(k)
    with pytest.raises(RuntimeError):
        B.check_resource_usage({"s": {"VGPRs Spill": "3"}})


def _built_report():
    if not os.path.exists(B.RESOURCE_REPORT):
        pytest.skip("no resource report: the library has not been built here")
    kernels, cur = {}, None
    with open(B.RESOURCE_REPORT) as f:
        for line in f:
            if not line.startswith(" "):
                cur = kernels.setdefault(line.strip(), {})
            else:
                a, b = line.strip().rsplit(": ", 1)
                cur[a] = b
    return kernels


def test_built_kernels_use_no_scratch_and_keep_occupancy():
    kernels = _built_report()
    dec = [k for k in kernels if "decode_split" in k]
    # (FP8 + static FP8 + INT8 + BF16) x 2 head dims + KIVI and KIVI with fp16 metadata (2 bit widths
    # x 2 head dims x 2 groups) + INT4 and Hadamard INT4 (groups 32, 64, 128 at d 128; 32, 64 at
    # d 64), for 2 input types, each as the plain decode and as the fused append + decode step
    assert len(dec) == 136
    B.check_resource_usage(kernels)
    for k in dec:
        assert int(kernels[k]["Occupancy [waves/SIMD]"]) >= 2, k
