"""Register and scratch budgets of the device kernels, read from the compiler's
resource report that the last build wrote (``iterative_stencil_pde_amd/build.py``
compiles every device translation unit with -Rpass-analysis=kernel-resource-usage
and keeps the merged result next to its objects, with a hash of the sources).
No GPU needed.

Every kernel must need no scratch: no register spills, no stack. A spill in the
persistent kernel is a per-lane memory round trip in whatever loop it lands in,
and its private segment has to be set up at launch ("Grid-Wide Barriers", the
residency requirement: the whole grid is resident, so every block pays for the
largest register demand of its kernel). The tile instances run 1024-thread
blocks and must stay within 128 VGPRs (four waves a SIMD); the streaming
instances run 512-thread blocks and must stay within 256.
"""

import json
import os
import re

import pytest

from iterative_stencil_pde_amd import build

LAYOUT = {"1": "stream", "2": "resident", "3": "register"}


def persistent_instance(mangled):
    """(element type, has b, layout, rows per wave, traced) of a pk_persistent
    instance, else None."""
    m = re.search(r"pk_persistentI([fd])Lb([01])ELi([123])ELi(\d+)ELb([01])E", mangled)
    if not m:
        return None
    return ("float" if m.group(1) == "f" else "double", m.group(2) == "1", LAYOUT[m.group(3)],
            int(m.group(4)), m.group(5) == "1")


def expected_instances():
    out = set()
    for t in ("float", "double"):
        for b in (False, True):
            out.add((t, b, "stream", 0, False))
            for traced in (False, True):
                out.add((t, b, "resident", 0, traced))
                for rows in (2, 4):
                    out.add((t, b, "register", rows, traced))
    return out


@pytest.fixture(scope="module")
def report():
    if not os.path.exists(build.RESOURCE_REPORT):
        pytest.skip("no resource report: build the library first")
    with open(build.RESOURCE_REPORT) as f:
        rep = json.load(f)
    assert rep["sources_sha"] == build.sources_sha(), \
        "the resource report is older than the device sources: rebuild (__graft_entry__.build())"
    return rep["kernels"]


def test_report_lists_every_persistent_instance(report):
    found = {persistent_instance(k) for k in report} - {None}
    assert found == expected_instances()


def test_report_covers_the_launch_kernels(report):
    for name in ("pk_sweep_launch", "pk_residual_launch", "pk_residual_finalize", "pk_scale_source"):
        assert any(name in k for k in report), name


def test_no_kernel_needs_scratch(report):
    for name, r in report.items():
        assert r.get("scratch", 0) == 0, (name, r)
        assert r.get("vgpr_spill", 0) == 0, (name, r)


def test_register_budgets(report):
    for name, r in report.items():
        inst = persistent_instance(name)
        if inst is None:
            continue
        limit = 256 if inst[2] == "stream" else 128
        assert r["vgpr"] <= limit, (inst, r)


def test_parser_reads_the_remarks():
    text = """x.hip:1:1: remark: Function Name: _ZN12_GLOBAL__N_113pk_persistentIdLb1ELi1ELi0ELb0EEEv8pk_kargs [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     TotalSGPRs: 98 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs: 235 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     SGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]"""
    got = build.parse_resource_usage(text)
    assert got == {"_ZN12_GLOBAL__N_113pk_persistentIdLb1ELi1ELi0ELb0EEEv8pk_kargs":
                   {"sgpr": 98, "vgpr": 235, "scratch": 0, "sgpr_spill": 3, "vgpr_spill": 0}}
    assert persistent_instance(next(iter(got))) == ("double", True, "stream", 0, False)
    assert persistent_instance("_ZN12_GLOBAL__N_113pk_persistentIfLb0ELi3ELi4ELb1EEEv8pk_kargs") == \
        ("float", False, "register", 4, True)
