"""Compiler resource guard (CPU): no kernel of libtg.so spills.

The GEMM kernels keep large accumulator and fragment arrays in registers and
rely on register-pressure measures (an in-place fragment refill, a slot
offset hidden from loop strength reduction) to fit them; a change that
breaks one of those shows up as scratch memory in the compiler's
kernel-resource-usage report, which the build collects for every kernel.
"""

import json
import os

import pytest

from dense_gemm_epilogues_tiled_amd import build as tg_build

SAMPLE = """\
csrc/x.hip:30:1: remark: Function Name: _ZN2tg3fooEv [-Rpass-analysis=kernel-resource-usage]
   30 | __global__ void foo() {
      | ^
csrc/x.hip:30:1: remark:     TotalSGPRs: 64 [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:30:1: remark:     VGPRs: 116 [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:30:1: remark:     AGPRs: 4 [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:30:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:30:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:30:1: remark:     Occupancy [waves/SIMD]: 4 [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:30:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:30:1: remark:     VGPRs Spill: 2 [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:30:1: remark:     LDS Size [bytes/block]: 1024 [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:9:1: remark: Function Name: _ZN2tg3barEv [-Rpass-analysis=kernel-resource-usage]
csrc/x.hip:9:1: remark:     VGPRs: 3 [-Rpass-analysis=kernel-resource-usage]
"""


def test_parse_resource_remarks():
    r = tg_build.parse_resource_remarks(SAMPLE)
    assert r["_ZN2tg3fooEv"] == {"sgprs": 64, "vgprs": 116, "agprs": 4, "scratch_bytes": 8, "dynamic_stack": False,
                                 "occupancy": 4, "sgpr_spill": 0, "vgpr_spill": 2, "lds_bytes": 1024}
    assert r["_ZN2tg3barEv"] == {"vgprs": 3}


def _resources():
    srcs = [os.path.join(tg_build.CSRC, f) for f in os.listdir(tg_build.CSRC)]
    newest = max(os.path.getmtime(p) for p in srcs)
    if not os.path.exists(tg_build.RESOURCES) or os.path.getmtime(tg_build.RESOURCES) < newest:
        tg_build.build()  # nothing built, or built from older sources
    with open(tg_build.RESOURCES) as f:
        return json.load(f)


def test_no_kernel_uses_scratch():
    res = _resources()
    kernels = {n: r for n, r in res.items() if "tg::" in r.get("demangled", n)}
    # every kernel family of the library is in the report
    for fam in ("gemm_tile_kernel", "gemm_ksplit_kernel", "gemm_softmax_kernel", "gemm_softmax_lds_kernel",
                "vector_add_kernel", "row_softmax_kernel", "attention_fwd_kernel", "count_mismatch_kernel"):
        assert any(fam + "<" in r["demangled"] or fam + "(" in r["demangled"] for r in kernels.values()), fam
    bad = {r["demangled"]: r for r in kernels.values()
           if r.get("scratch_bytes", 1) != 0 or r.get("vgpr_spill", 1) != 0 or r.get("sgpr_spill", 1) != 0
           or r.get("dynamic_stack", True)}
    assert not bad, f"kernels with scratch / spills: {json.dumps(bad, indent=1)}"
    for r in kernels.values():
        assert r["vgprs"] + r["agprs"] <= 512 and r["lds_bytes"] <= 160 * 1024, r["demangled"]
