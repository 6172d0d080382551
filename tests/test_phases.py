"""CPU: the phase-stamp summary of the profiling tool.  Stamps are ticks of
the 100 MHz constant clock; a 0 is a phase a workgroup did not pass (the
second pass of a one-pass attention workgroup) and a row of zeros a
workgroup the launch did not have."""

import numpy as np

from dense_gemm_epilogues_tiled_amd import phases


def _parse(lines):
    rows = {}
    for line in lines[1:-1]:
        name = line[:28].strip()
        vals = line[28:].split()
        rows[name] = [float(v) for v in vals]
    return rows


def test_summary_of_complete_stamps():
    names = [f"p{i}" for i in range(8)]
    # two workgroups, 1 us (100 ticks) between phases, the second starting 0.5 us later
    base = np.arange(8, dtype=np.uint64) * 100 + 1000
    stamps = np.stack([base, base + 50])
    lines = phases.summarize(stamps, names)
    rows = _parse(lines)
    assert rows["p0"][:3] == [0.0, 0.25, 0.5]      # min / median / max from the first start
    assert rows["p7"][:3] == [7.0, 7.25, 7.5]
    assert rows["p3"][3] == 1.0                     # median duration of a phase
    assert rows["p3"][4] == 2                       # workgroups that passed it
    assert lines[-1].strip().startswith("span") and "7.500 us over 2 workgroups" in lines[-1]


def test_missing_phases_and_absent_workgroups_are_skipped():
    names = [f"p{i}" for i in range(8)]
    one_pass = np.array([1000, 1100, 1200, 1300, 0, 0, 0, 0], dtype=np.uint64)
    two_pass = np.array([1000, 1100, 1200, 1300, 1300, 1400, 1500, 1600], dtype=np.uint64)
    absent = np.zeros(8, dtype=np.uint64)
    lines = phases.summarize(np.stack([one_pass, two_pass, absent]), names)
    rows = _parse(lines)
    assert rows["p3"][4] == 2 and rows["p5"][4] == 1   # the second pass counts one workgroup
    assert rows["p5"][:3] == [4.0, 4.0, 4.0] and rows["p5"][3] == 1.0
    assert "over 2 workgroups" in lines[-1]             # the all-zero row is not a workgroup


def test_every_instrumented_kernel_has_eight_phases_and_a_reader():
    for kernel, names in phases.PHASES.items():
        assert len(names) == 8, kernel
        assert phases.READER[kernel].startswith("tg_phases_")
