"""The build's register and scratch check (CPU only): the compiler's
resource remarks are parsed, and a kernel that spills to scratch fails the
build unless its shape has a listed reason."""
import pytest

from vocab_softmax_cross_amd import build as B

HEADLINE = "_ZN4vsce12_GLOBAL__N_121fused_resident_kernelILi1ELi1024ELi11ELi5ELi5056ELi0ELb0ELb0ELi8EEEvNS_7RowArgsE"
WEIGHTED = "_ZN4vsce12_GLOBAL__N_121fused_resident_kernelILi1ELi1024ELi11ELi5ELi5056ELi0ELb1ELb0ELi8EEEvNS_7RowArgsE"

REMARKS = f"""In file included from x.hip:2:
x.h:53:1: remark: Function Name: {HEADLINE} [-Rpass-analysis=kernel-resource-usage]
   53 | void fused_resident_kernel(const RowArgs a) {{
      | ^
x.h:53:1: remark:     VGPRs: 62 [-Rpass-analysis=kernel-resource-usage]
x.h:53:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.h:53:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.h:53:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:3: warning: something else the compiler said
"""


def test_remarks_are_parsed_and_separated_from_other_output():
    kernels, rest = B._resources(REMARKS)
    assert kernels == [{"name": HEADLINE, "VGPRs": "62", "ScratchSize [bytes/lane]": "0",
                        "VGPRs Spill": "0", "Occupancy [waves/SIMD]": "8"}]
    assert rest.strip() == "x.hip:9:3: warning: something else the compiler said"


def test_listed_shapes_have_reasons_and_the_headline_has_none():
    assert B.scratch_reason(WEIGHTED)
    assert B.scratch_reason(HEADLINE) is None
    assert B.scratch_reason("_ZN4vsce12_GLOBAL__N_114gemm_nt_kernelILi0E") is None


def test_unlisted_scratch_fails_the_build(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "REPORT", str(tmp_path / "report.txt"))
    ok = {"name": WEIGHTED, "source": "fused_bf16.hip", "ScratchSize [bytes/lane]": "20"}
    B.check_resources([ok])
    bad = {"name": HEADLINE, "source": "fused_bf16.hip", "ScratchSize [bytes/lane]": "4"}
    with pytest.raises(RuntimeError, match="without a listed reason"):
        B.check_resources([ok, bad])
    assert HEADLINE in (tmp_path / "report.txt").read_text()
