"""HBM-traffic summariser (dense_gemm_epilogues_tiled_amd/traffic.py) on
synthetic rocprofv3 counter files: counter units are calibrated by the copy
kernel's reading, per-dispatch values are summed over counter instances, and
the workload kernel's median dispatch is taken."""

import csv
import os

import pytest

from dense_gemm_epilogues_tiled_amd import traffic

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
GEMM = "void tg::gemm_tile_kernel<128, 128, 64, 2, 4, 4, true, false, tg::F16>(tg::GemmParams)"


def _write(directory, counter, rows):
    os.makedirs(os.path.join(directory, "host"), exist_ok=True)
    with open(os.path.join(directory, "host", "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, values) in enumerate(rows):
            for v in values:  # one row per counter instance
                w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})


def test_read_counter_sums_instances_per_dispatch(tmp_path):
    _write(str(tmp_path), "FETCH_SIZE", [("__amd_rocclr_copyBuffer", [100.0, 28.0]), (GEMM, [1.0, 2.0, 3.0])])
    got = traffic.read_counter(str(tmp_path), "FETCH_SIZE")
    assert got == {"__amd_rocclr_copyBuffer": [128.0], GEMM: [6.0]}
    assert traffic.read_counter(str(tmp_path), "WRITE_SIZE") == {}


def test_measure_scales_by_the_copy(tmp_path):
    copy_kib = traffic.COPY_MIB * 1024
    f, w = str(tmp_path / "f"), str(tmp_path / "w")
    # the copy reads half its true size in FETCH_SIZE units and all of it in WRITE_SIZE units;
    # three GEMM dispatches, the median one counts
    _write(f, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", [copy_kib / 4, copy_kib / 4]), (GEMM, [10000.0]),
                             (GEMM, [24000.0, 600.0]), (GEMM, [90000.0])])
    _write(w, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", [copy_kib]), (GEMM, [8192.0]), (GEMM, [8192.0]),
                             (GEMM, [8192.0])])
    rec = traffic.measure("C3", f, w)
    assert rec["kernel"] == GEMM
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == pytest.approx(24600.0 * 2 * 1024)
    assert rec["write_bytes"] == pytest.approx(8192.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(rec["fetch_bytes"] + rec["write_bytes"])
    # fp16 A, B and C of 2048 x 2048, bias of 2048
    assert rec["algorithmic_bytes"] == 3 * 2048 * 2048 * 2 + 2048 * 2


def test_missing_kernel_is_an_error(tmp_path):
    _write(str(tmp_path), "FETCH_SIZE", [("__amd_rocclr_copyBuffer", [1.0])])
    with pytest.raises(LookupError):
        traffic.measure("C3", str(tmp_path), str(tmp_path))
