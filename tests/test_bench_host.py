"""Host-side behaviour of bench.py (no GPU): it refuses more than one GPU with
a message and exit status 2, and names the kernel a tile configuration
launches the way the kernel trace does."""

import os
import subprocess
import sys

import dense_gemm_epilogues_tiled_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_kernel_names_follow_the_configuration():
    names = {}
    for c in tg.configs():
        names[c["id"]] = bench.kernel_name(c)
        if c["kind"] == tg.TG_KERNEL_GEMM_SOFTMAX:
            assert names[c["id"]] in ("gemm_softmax_kernel", "gemm_softmax_lds_kernel")
        elif c["waves"] == 2 * c["wave_m"] * c["wave_n"]:
            assert names[c["id"]] == "gemm_ksplit_kernel"
        else:
            assert c["waves"] == c["wave_m"] * c["wave_n"] and names[c["id"]] == "gemm_tile_kernel"
    assert "gemm_ksplit_kernel" in names.values() and "gemm_tile_kernel" in names.values()
