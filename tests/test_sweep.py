"""CPU tests of the offline sweep's bookkeeping (no GPU): the fastest valid
candidate per workload, the generated config_table.inc (it compiles with the
table entry type api.cpp uses, and round-trips the chosen ids), the results
file bound to the kernel sources, and the scratch-memory filter."""

import json
import os
import re
import subprocess

import pytest

import dense_gemm_epilogues_tiled_amd as tg
from dense_gemm_epilogues_tiled_amd import sweep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _results():
    return {
        "C3": {"11/2/0": {"id": 11, "group_m": 2, "xcd_remap": 0, "valid": True, "us": 20.1, "tflops": 855.0},
               "10/8/1": {"id": 10, "group_m": 8, "xcd_remap": 1, "valid": True, "us": 19.9, "tflops": 863.0},
               "3/4/0": {"id": 3, "group_m": 4, "xcd_remap": 0, "valid": False, "frob": 0.5}},
        "C2": {"11/2/0": {"id": 11, "group_m": 2, "xcd_remap": 0, "valid": True, "us": 18.7, "tflops": 919.0}},
        "C5": {"17/1/0": {"id": 17, "group_m": 1, "xcd_remap": 0, "valid": True, "us": 7.8, "tflops": 137.0},
               "15/1/0": {"id": 15, "group_m": 1, "xcd_remap": 0, "valid": True, "us": 9.9, "tflops": 108.0}},
        "C4a": {"4/4/1": {"id": 4, "group_m": 4, "xcd_remap": 1, "valid": False, "frob": 1.0}},
    }


def test_best_per_workload_takes_the_fastest_valid_row():
    best = sweep.best_per_workload(_results())
    assert best["C3"]["id"] == 10 and best["C3"]["group_m"] == 8
    assert best["C5"]["id"] == 17
    assert "C4a" not in best  # no valid row


def test_written_table_compiles_and_round_trips(tmp_path):
    best = sweep.best_per_workload(_results())
    path = tmp_path / "config_table.inc"
    sweep.write_table(best, str(path))
    text = path.read_text()
    # C2 and C3 share a key (fp16, row-major B, elementwise, 2048^3): the headline C3 decides
    rows = re.findall(r"\{(TG_DTYPE_\w+), (\d), (\d), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\},\s*// (\w+)", text)
    got = {r[9]: (r[0], int(r[6]), int(r[7]), int(r[8])) for r in rows}
    assert got == {"C3": ("TG_DTYPE_F16", 10, 8, 1), "C5": ("TG_DTYPE_F16", 17, 1, 0)}
    # the same entry type as api.cpp, compiled with the host compiler
    src = tmp_path / "t.cpp"
    src.write_text(f'#include "tg.h"\n#include <stdint.h>\nstruct TableEntry {{ int dtype, b_col_major, epilogue_kind; '
                   f'int64_t M, N, K; int variant, group_m, xcd_remap; }};\n#include "{path}"\n'
                   f"int main() {{ return (int)(sizeof(kTable) / sizeof(kTable[0])) == 2 ? 0 : 1; }}\n")
    exe = tmp_path / "t"
    r = subprocess.run(["g++", "-std=c++17", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert subprocess.run([str(exe)]).returncode == 0


def test_results_from_other_kernel_sources_are_discarded(tmp_path):
    path = tmp_path / "res.json"
    path.write_text(json.dumps({"kernel_source_sha": sweep.kernel_source_sha(), "workloads": _results()}))
    assert sweep.load_results(str(path)) == _results()
    path.write_text(json.dumps({"kernel_source_sha": "0" * 16, "workloads": _results()}))
    assert sweep.load_results(str(path)) == {}
    path.write_text(json.dumps(_results()))  # a file without the stamp
    assert sweep.load_results(str(path)) == {}
    assert sweep.load_results(str(tmp_path / "missing.json")) == {}
    assert sweep.DEFAULT_RESULTS.startswith(os.path.realpath(os.sep)) and "_work" not in sweep.DEFAULT_RESULTS


def test_every_configuration_names_its_kernels_and_spills_are_filtered():
    from dense_gemm_epilogues_tiled_amd import build as tg_build
    if not os.path.exists(tg_build.RESOURCES):
        pytest.skip("no build report: run python -m dense_gemm_epilogues_tiled_amd.build")
    with open(tg_build.RESOURCES) as f:
        res = json.load(f)
    names = [r["demangled"] for r in res.values()]
    for c in tg.configs():
        pre = sweep.kernel_prefix(c)
        assert any(n.startswith(pre) for n in names), (c, pre)
    assert sweep.spilling_configs(res, tg.configs()) == set()
    # a planted spill in one instance marks that configuration only
    victim = tg.configs()[4]
    key = next(k for k, r in res.items() if r["demangled"].startswith(sweep.kernel_prefix(victim)))
    res[key] = dict(res[key], scratch_bytes=64)
    assert sweep.spilling_configs(res, tg.configs()) == {4}
