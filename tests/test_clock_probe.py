"""GPU: the shader-clock probe reads a plausible clock under MFMA load, and
its constant counter runs at ~100 MHz against the host clock."""

import pytest

tg = pytest.importorskip("dense_gemm_epilogues_tiled_amd")

pytestmark = pytest.mark.gpu


def test_clock_under_mfma_load_is_plausible():
    r = tg.shader_clock_mhz(blocks=1024, iters=300000)
    print(f"[clock] {r}", flush=True)
    assert 500.0 <= r["mhz"] <= 2600.0          # gfx950 shader clock range
    # the ticks of the slowest workgroup cannot exceed the host-measured window;
    # launch overhead makes the ratio a lower bound of the counter's rate
    assert 80.0 <= r["realtime_mhz_vs_host"] <= 101.0
    assert r["peak_tflops_at_clock"] == pytest.approx(256 * 4096 * r["mhz"] / 1e6)
