"""The build's kernel resource check (no GPU): every kernel must compile
without private memory, read from the compiler's kernel-resource-usage
remarks."""
import os
import subprocess

import pytest

from global_gqa_attention_kv_amd import build as b

REMARKS = """\
x.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs: 9 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 400 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
"""


def test_parse_and_reject():
    res = b.kernel_resources(REMARKS)
    assert res == {
        "kern_a": {"ScratchSize [bytes/lane]": 0, "SGPRs Spill": 0,
                   "VGPRs Spill": 0},
        "kern_b": {"ScratchSize [bytes/lane]": 400, "SGPRs Spill": 0,
                   "VGPRs Spill": 3}}
    b.check_resources({"kern_a": res["kern_a"]}, "x.hip")
    with pytest.raises(RuntimeError, match="kern_b"):
        b.check_resources(res, "x.hip")


def test_library_kernels_use_no_private_memory(tmp_path):
    """The append kernels and the fp8-to-bf16 copy compiled as the build
    compiles them (the build applies the same check to every source)."""
    src = os.path.join(b.CSRC, "kv_append.hip")
    r = subprocess.run([b.HIPCC] + b.COMMON + b.DEVICE + b.RESOURCES +
                       ["-c", src, "-o", str(tmp_path / "a.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    res = b.kernel_resources(r.stderr)
    assert len(res) == 3, res
    b.check_resources(res, src)
