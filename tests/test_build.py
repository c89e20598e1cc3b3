"""The build's spill check reads the compiler's kernel-resource-usage remarks."""

import pytest

from fp8_quantized_skinny_amd import build

REPORT = """\
a.hip:10:1: remark: Function Name: _Zk1 [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     VGPRs: 62 [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark: Function Name: _Zk2 [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark:     ScratchSize [bytes/lane]: 24 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_sizes_per_kernel():
    assert build.scratch_per_kernel(REPORT) == {"_Zk1": 0, "_Zk2": 24}


def test_a_new_spill_fails_the_build(monkeypatch):
    monkeypatch.setattr(build, "KNOWN_SPILLS", {})
    with pytest.raises(RuntimeError, match="_Zk2"):
        build.check_spills(build.scratch_per_kernel(REPORT), "a.hip")


def test_a_known_spill_passes_unless_it_grows(monkeypatch):
    monkeypatch.setattr(build, "KNOWN_SPILLS", {"_Zk2": 24})
    build.check_spills(build.scratch_per_kernel(REPORT), "a.hip")
    monkeypatch.setattr(build, "KNOWN_SPILLS", {"_Zk2": 16})
    with pytest.raises(RuntimeError):
        build.check_spills(build.scratch_per_kernel(REPORT), "a.hip")
