"""GPU: the register layouts the kernels rely on, read back from the
hardware with tg_layout_probe and checked against the formulas the kernel
sources state (device.hpp: mfma16x16x32, lds_read_tr8).

  * v_mfma_f32_16x16x32_{f16,bf16}: operand lane l holds row (first operand)
    or column (second operand) l % 16 and 8 k values of k-group l / 16, in the
    same k order for both operands; accumulator lane l holds column l % 16,
    rows 4 (l / 16) + r.  With the first operand one-hot at (lane la,
    element ea), accumulator register la % 4 of lanes 16 ((la % 16) / 4) + j
    holds the second operand's element ea of lane j + 16 (la / 16), and every
    other output is zero.
  * ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
    i % 4 of the four 16-bit values addressed by lanes i/4, 4 + i/4, 8 + i/4,
    12 + i/4 of the group.
"""

import numpy as np
import pytest
import torch

tg = pytest.importorskip("dense_gemm_epilogues_tiled_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _code(kind, v):
    v = np.asarray(v)
    return (v + 1.0) if kind == 0 else (16.0 + (v % 16)) * np.exp2(v // 16)


@pytest.mark.parametrize("kind", [0, 1], ids=["f16", "bf16"])
def test_mfma_16x16x32_layout(kind):
    tg.load(build_if_missing=False)
    out = torch.full((512, 64, 4), float("nan"), dtype=torch.float32, device=DEV)
    assert tg.tg_layout_probe(kind, out.data_ptr(), torch.cuda.current_stream().cuda_stream) == tg.TG_OK
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = np.zeros((512, 64, 4))
    for la in range(64):
        for ea in range(8):
            row = la % 16
            for j in range(16):
                want[8 * la + ea, 16 * (row // 4) + j, row % 4] = _code(kind, 8 * (j + 16 * (la // 16)) + ea)
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]


def test_transposing_lds_read_lane_map():
    tg.load(build_if_missing=False)
    out = torch.full((64, 4), -1, dtype=torch.int32, device=DEV)
    assert tg.tg_layout_probe(2, out.data_ptr(), torch.cuda.current_stream().cuda_stream) == tg.TG_OK
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = np.zeros((64, 4), dtype=np.int64)
    for lane in range(64):
        g, i = lane // 16, lane % 16
        for e in range(4):
            src_lane = 16 * g + 4 * e + i // 4  # lane whose 4 values it draws from
            want[lane, e] = 4 * src_lane + i % 4  # value index = byte address / 2
    assert np.array_equal(got, want), (got[:4], want[:4])


def test_probe_rejects_bad_arguments():
    tg.load(build_if_missing=False)
    assert tg.tg_layout_probe(3, 16, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_layout_probe(0, None, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_layout_probe(0, 8, None) == tg.TG_ERR_MISALIGNED
