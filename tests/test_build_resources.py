"""The build's register check: the compiler's resource-usage remarks are
parsed per kernel, and a kernel with scratch memory or vector-register spills
fails the build (such a kernel once made the fused append-and-decode step
40 % slower with no change in its results)."""
import os

import pytest

from decode_attention_select_amd import build

SAMPLE = """\
x.hip:22:1: remark: Function Name: _ZN3kvq1aEv [-Rpass-analysis=kernel-resource-usage]
   22 | void a() {
      | ^
x.hip:22:1: remark:     VGPRs: 76 [-Rpass-analysis=kernel-resource-usage]
x.hip:22:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:22:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:22:1: remark:     SGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]
x.hip:40:1: remark: Function Name: _ZN3kvq1bEv [-Rpass-analysis=kernel-resource-usage]
x.hip:40:1: remark:     VGPRs: 255 [-Rpass-analysis=kernel-resource-usage]
x.hip:40:1: remark:     ScratchSize [bytes/lane]: 224 [-Rpass-analysis=kernel-resource-usage]
x.hip:40:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:60:1: remark: Function Name: _ZN3kvq1cEv [-Rpass-analysis=kernel-resource-usage]
x.hip:60:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:60:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
"""


def test_remarks_parse_per_kernel():
    rows = build._resource_rows(SAMPLE)
    assert [n for n, _ in rows] == ["_ZN3kvq1aEv", "_ZN3kvq1bEv", "_ZN3kvq1cEv"]
    assert rows[0][1]["VGPRs"] == "76" and rows[1][1]["ScratchSize [bytes/lane]"] == "224"


def test_scratch_and_vector_spills_are_flagged_scalar_spills_are_not():
    assert build.check_resources(build._resource_rows(SAMPLE)) == ["_ZN3kvq1bEv", "_ZN3kvq1cEv"]


def test_report_round_trips(tmp_path):
    rows = build._resource_rows(SAMPLE)
    build.write_resources(rows, str(tmp_path / "r.txt"))
    back = build.read_resources(str(tmp_path / "r.txt"))
    assert [n for n, _ in back] == [n for n, _ in rows]
    assert build.check_resources(back) == ["_ZN3kvq1bEv", "_ZN3kvq1cEv"]


def test_built_library_has_no_scratch():
    if not os.path.exists(build.RESOURCES):
        pytest.skip("no resource report: the library was not built here")
    rows = build.read_resources()
    assert any(n.startswith("_ZN3kvq13decode_kernel") for n, _ in rows)
    assert build.check_resources(rows) == []
